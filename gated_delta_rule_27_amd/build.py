"""Build libkda.so (HIP, gfx950) in-tree.

``python -m gated_delta_rule_27_amd.build`` or ``build()`` compiles the
kernels and the C ABI in ``csrc/`` with hipcc for gfx950 into
``gated_delta_rule_27_amd/libkda.so``.  Each source is compiled to an object
in parallel, then linked.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libkda.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["kda_api.cpp", "kda_chunk.hip", "kda_chunk_ws2.hip", "kda_chunk_ws2_s2.hip", "kda_chunk_ws3.hip",
           "kda_decode.hip", "kda_decode_multi.hip",
           "kda_segment.hip", "kda_layer.hip", "kda_bwd.hip",
           "kda_bwd_ws.hip", "kda_noalloc.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 VALU forms are kept out of the generated code.
COMMON = ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-result"]
# per-source additions: the half-head prefill with outputs and the
# single-step decode are scheduled by LLVM's iterative ILP strategy (faster
# there; slower or spilling for the other variants of the prefill kernel
# and for the multi-token decode, which stay with the default)
EXTRA = {"kda_chunk_ws2_s2.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
         "kda_decode.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]}


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + EXTRA.get(src, []) + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise subprocess.CalledProcessError(r.returncode, cmd)
    return obj


def build(verbose=False):
    """Compile every source for gfx950 and link libkda.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, LIB)
    return LIB


def resource_usage(src):
    """Per-kernel register and scratch use of one HIP source, from the
    compiler's resource-usage remarks: {kernel symbol: {"vgpr", "agpr",
    "scratch", "occupancy"}} (scratch in bytes per lane; non-zero means
    spills or a stack)."""
    import re
    cmd = [HIPCC] + COMMON + EXTRA.get(src, []) + ["-x", "hip", "--cuda-device-only", "-c", os.path.join(CSRC, src),
                              "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise subprocess.CalledProcessError(r.returncode, cmd)
    out, cur = {}, None
    keys = {"VGPRs": "vgpr", "AGPRs": "agpr", "ScratchSize [bytes/lane]": "scratch",
            "Occupancy [waves/SIMD]": "occupancy"}
    for line in r.stderr.splitlines():
        m = re.search(r"remark:\s+(.*?): (\S+) \[-Rpass-analysis", line)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None and key in keys:
            cur[keys[key]] = int(val)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
