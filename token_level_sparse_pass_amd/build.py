"""Builds libhs2.so (the Hybrid Block engine) with hipcc for gfx950, in-tree.

    python -m token_level_sparse_pass_amd.build [-v]
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libhs2.so")
SOURCES = ["hs2_api.hip", "attn_fwd.hip", "attn_fwd_bf16.hip", "attn_decode_bf16.hip",
           "score.hip", "score_bf16.hip",
           "select.hip", "kv_append.hip", "kv_bridge.hip",
           "sparse_attn.hip", "sparse_attn_bf16.hip", "attn_bwd.hip", "attn_bwd_bf16.hip",
           "sparse_bwd.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         # packed fp32 math stays off: plain scalar/float2 code only
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # MFMA results and accumulators in ordinary VGPRs: otherwise the
         # compiler parks some kernels' accumulators in AGPRs and copies them
         # to VGPRs and back on every loop trip around a VALU rescale (the
         # sparse layers, decode pass 1); kernels that use no AGPRs compile
         # to the same code either way
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-I", INCLUDE, "-I", CSRC]
# per-source additions: the bf16 pass-1 and sparse-layer kernels take their
# row maxima with plain max instructions, which fmaxf emits only when NaNs
# need no handling (their logits are finite or -inf)
EXTRA = {"attn_fwd_bf16.hip": ["-fno-honor-nans"], "attn_decode_bf16.hip": ["-fno-honor-nans"],
         "sparse_attn_bf16.hip": ["-fno-honor-nans"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(line for line in (r.stderr or "").splitlines()
                     if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if verbose and errs.strip():
        print(errs)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libhs2.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
