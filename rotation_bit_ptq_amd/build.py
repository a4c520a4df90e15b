"""Builds liborbit.so (the C-ABI library) in-tree for gfx950 with hipcc."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "liborbit.so")
# measured roofline ceilings for bench.py (not part of the layer's C ABI)
PEAKS_SOURCES = ["peaks.hip"]
PEAKS_OUT = os.path.join(HERE, "libpeaks.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["abi.cpp", "codebook.cpp", "rpbh_quant.hip", "rpbh_bf16_act.hip",
           "rpbh_bf16_weight.hip", "rpbh_bf16_plain.hip", "rpbh_f32.hip",
           "rpbh_fast_a64.hip", "rpbh_fast_a128.hip", "rpbh_fast_a256.hip",
           "rpbh_fast_w64.hip", "rpbh_fast_w128.hip", "rpbh_fast_w256.hip",
           "rpbh_fast_r64.hip", "rpbh_fast_r128.hip", "rpbh_fast_r256.hip",
           "rpbh_mfma_a64.hip", "rpbh_mfma_a128.hip", "rpbh_mfma_a256.hip", "rpbh_mfma_w64.hip",
           "rpbh_mfma_w128.hip", "rpbh_mfma_w256.hip", "rpbh_mfma_r.hip",
           "rpbh_m2_a128.hip", "rpbh_m2_a256.hip", "rpbh_m2_w128.hip", "rpbh_m2_w256.hip",
           "rpbh_m2_r.hip", "rpbh_m2_big.hip", "qgemm.hip", "qgemm_int8.hip",
           "qgemm_a2.hip", "qgemm_a3.hip", "qgemm_a4.hip", "qgemm_a6.hip", "qgemm_a8.hip"]
# Packed fp32 VALU instructions are kept out of the generated code.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def _newest_header():
    inc = os.path.join(os.path.dirname(HERE), "include")
    paths = [os.path.join(d, f) for d in (CSRC, inc) if os.path.isdir(d)
             for f in os.listdir(d) if f.endswith(".h")]
    return max((os.path.getmtime(p) for p in paths), default=0.0)


def _compile(src, objdir, incremental=False, headers_mtime=0.0):
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    if incremental and os.path.exists(obj):
        t = os.path.getmtime(obj)
        if t > os.path.getmtime(os.path.join(CSRC, src)) and t > headers_mtime:
            return obj
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=False, incremental=False):
    """Compiles every source (incremental=True: only those whose object is
    older than the source or any header) and links liborbit.so."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    hdr = _newest_header()
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, objdir, incremental, hdr), SOURCES))
    _link(objs, OUT)
    _link([_compile(s, objdir, incremental, hdr) for s in PEAKS_SOURCES], PEAKS_OUT)
    if verbose:
        print(f"built {OUT} and {PEAKS_OUT}")
    return OUT


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {out} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv)
    sys.exit(0)
