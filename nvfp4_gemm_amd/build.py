"""Build libpact.so (hand-written HIP for gfx950) in-tree with hipcc.

    python -m nvfp4_gemm_amd.build        # or nvfp4_gemm_amd.build.build()

Every source is compiled for gfx950 only, with IEEE-exact binary32 division
and square root, denormals kept, no floating-point contraction, and packed
FP32 instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpact.so")
SOURCES = ["pact_api.hip", "pact_quant.hip", "pact_layout.hip", "pact_gemm.hip", "pact_lora_grad.hip",
           "pact_optim.hip", "pact_gptq.hip", "pact_diag.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, "-I", BUILD, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _sigmoid_table() -> None:
    """Generates the SiLU kernels' sigma32 and dsilu32 tables (a host program run at build time)."""
    exe = os.path.join(BUILD, "gen_sigmoid_table")
    cmd = [os.environ.get("CXX", "g++"), "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
           os.path.join(CSRC, "gen_sigmoid_table.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"table generator build failed:\n{r.stderr}")
    r = subprocess.run([exe, os.path.join(BUILD, "pact_sigmoid_table.inc"),
                        os.path.join(BUILD, "pact_dsilu_table.inc")], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"table generator failed:\n{r.stderr}")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    _sigmoid_table()
    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
