"""Build the gfx950 shared library ``libsv.so`` in-tree with hipcc.

``python draft_token_verification_sv_amd/build.py`` (or ``build()``) compiles
every source under ``csrc/`` to an object file in parallel and links them.
``--debug`` (``build(debug=True)``) builds ``libsv_debug.so`` instead: the
same kernels compiled with SV_DEBUG, which record broken device-side inputs
in the word that ``sv_check_device_errors`` returns.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libsv.so")
OUT_DEBUG = os.path.join(PKG, "libsv_debug.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["sv_api.cpp", "attn_dma.hip", "attn_mfma.hip", "attn_valu.hip", "attn_q4.hip", "attn_q4w.hip", "accept.hip",
           "compact.hip", "append.hip", "recurrent.hip", "topk.hip", "debug.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in VGPRs: the online softmax rescales them with
    # vector ALU ops, and the AGPR form made the compiler copy every
    # accumulator AGPR -> VGPR on each loop iteration
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-function",
]
# extra flags per source: the cooperative 4-bit kernel keeps no NaN semantics
# in its maxima (inputs are finite; masked scores are -inf, which stays exact)
EXTRA = {"attn_q4.hip": ["-fno-honor-nans"], "attn_q4w.hip": ["-fno-honor-nans"]}
# sources left to the compiler's own choice of accumulation registers (none:
# the cooperative 4-bit kernel places its O accumulators itself)
NO_VGPR_FORM: set = set()


def _compile(src: str, obj_dir: str, debug: bool) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    flags = [f for f in FLAGS if not (src in NO_VGPR_FORM and f in ("-mllvm", "-amdgpu-mfma-vgpr-form=1"))]
    cmd = [HIPCC, *flags, *EXTRA.get(src, []), *(["-DSV_DEBUG"] if debug else [])]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, debug: bool = False) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    out = OUT_DEBUG if debug else OUT
    obj_dir = os.path.join(PKG, "_build_debug" if debug else "_build")
    os.makedirs(obj_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir, debug), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    shutil.rmtree(obj_dir, ignore_errors=True)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True, debug="--debug" in sys.argv[1:])
    sys.exit(0)
