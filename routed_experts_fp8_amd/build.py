"""Build libmoefp8.so for gfx950 with hipcc (in-tree, no JIT cache).

Usage: python routed_experts_fp8_amd/build.py   (or __graft_entry__.build(); importing the
package first would load the library this script builds)

Every HIP source is compiled with:
  -ffp-contract=off                       a*b+c stays two roundings; the
                                          kernels write fused multiply-adds
                                          explicitly where they want them
  -fhip-fp32-correctly-rounded-divide-sqrt  IEEE binary32 division (the
                                          quantisation scale and codes depend
                                          on it)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                          no packed-fp32 instructions
"""

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libmoefp8.so")
BUILD_DIR = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["status.cpp", "quant.hip", "transpose.hip", "route.hip", "permute.hip", "route_permute.hip",
           "swiglu_combine.hip", "gemm.hip", "backward.hip", "wgrad.hip", "router.hip", "probe.hip"]

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-ffp-contract=off",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]
DEVICE_FLAGS = [
    f"--offload-arch={ARCH}",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD_DIR, src + ".o")
    cmd = [HIPCC] + FLAGS + ["-x", "hip"] + DEVICE_FLAGS + ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def build(verbose=False, jobs=None):
    """Compile every source and link libmoefp8.so next to this file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    if verbose:
        for (_, err), src in zip(results, SOURCES):
            msgs = [l for l in err.splitlines() if "packed-fp32-ops" not in l and l.strip()]
            if msgs:
                print(f"[{src}]\n" + "\n".join(msgs))
    objs = [o for o, _ in results]
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
