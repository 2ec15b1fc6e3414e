"""Build libtdf.so (gfx950) in-tree with hipcc.

    python -m transformer_decode_forward_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtdf.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

DEVICE_SOURCES = ["k_decode.hip", "k_attn_decode.hip", "k_gemm.hip", "k_attn_prefill.hip", "k_sample.hip", "k_skinny.hip", "k_kvq8.hip", "tdf_api.hip"]
HOST_SOURCES = ["host_plan.cpp"]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-x", "hip",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
# Decode attention: matrix-core accumulators in ordinary VGPRs.  With the
# default (AGPR accumulators) the compiler copies the 36 accumulator registers
# out and back around every tile, because the online-softmax rescale works on
# them with vector instructions.
EXTRA_FLAGS = {"k_attn_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC] + HIP_FLAGS + EXTRA_FLAGS.get(src, []) + ["-c", path, "-o", obj]
    else:
        cmd = ["g++"] + HOST_FLAGS + ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{msgs}")
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    sources = [s for s in DEVICE_SOURCES + HOST_SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
