"""Build libqlin.so (HIP for gfx950) in-tree with hipcc.

Each translation unit is compiled on its own (in parallel), then linked into
quantized_matmul_amd/libqlin.so. Flags:
  --offload-arch=gfx950 -O3           CDNA4 only
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                      no packed fp32 VALU instructions
  -ffp-contract=off (quant.hip)       bit-exact quantize/dequantize rounding
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_obj")
LIB = os.path.join(HERE, "libqlin.so")
SOURCES = ["qlin_api.cpp", "quant.hip", "qmm_generic.hip", "qmm_decode.hip", "qmm_tiled.hip", "qmm_nt.hip",
           "qmm_prefill.hip", "qmm_prefill2.hip", "gather_index.hip", "qqmm_mx8.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
          "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
PER_FILE = {"quant.hip": ["-ffp-contract=off"]}


def _compile(src):
    out = os.path.join(OBJ, src + ".o")
    cmd = [HIPCC, *COMMON, *PER_FILE.get(src, []), "-c", os.path.join(CSRC, src), "-o", out]
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    # keep warnings visible, minus hipcc's host-pass note about the gfx feature
    msg = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if msg:
        print(msg, file=sys.stderr)
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
