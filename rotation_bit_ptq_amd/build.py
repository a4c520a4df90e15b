"""Builds liborbit.so (the C-ABI library) in-tree for gfx950 with hipcc."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "liborbit.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["abi.cpp", "codebook.cpp", "rpbh_quant.hip", "rpbh_bf16_act.hip",
           "rpbh_bf16_weight.hip", "rpbh_bf16_plain.hip", "rpbh_f32.hip",
           "rpbh_fast_a64.hip", "rpbh_fast_a128.hip", "rpbh_fast_a256.hip",
           "rpbh_fast_w64.hip", "rpbh_fast_w128.hip", "rpbh_fast_w256.hip",
           "rpbh_fast_r64.hip", "rpbh_fast_r128.hip", "rpbh_fast_r256.hip",
           "rpbh_mfma_a64.hip", "rpbh_mfma_a128.hip", "rpbh_mfma_a256.hip", "rpbh_mfma_w64.hip",
           "rpbh_mfma_w128.hip", "rpbh_mfma_w256.hip", "rpbh_mfma_r.hip", "qgemm.hip", "qgemm_int8.hip",
           "qgemm_a2.hip", "qgemm_a3.hip", "qgemm_a4.hip", "qgemm_a6.hip", "qgemm_a8.hip"]
# Packed fp32 VALU instructions are kept out of the generated code.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def _compile(src, objdir):
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=False):
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, objdir), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
