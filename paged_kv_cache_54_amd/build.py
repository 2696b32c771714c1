"""Build libpa.so (gfx950) in-tree with hipcc.

Each source compiles to an object under paged_kv_cache_54_amd/_build/ in
parallel, then hipcc links the shared library next to this file.  All device
code is built with packed-FP32 instructions disabled.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["pa_api.cpp", "kv_append.hip", "decode_valu.hip", "decode_mfma.hip",
           "decode_mfma_append.hip", "decode_mfma_heads.hip", "decode_mfma_heads_append.hip",
           "decode_mfma_multi.hip", "merge.hip", "blocks.hip", "step_prep.hip", "cascade.hip",
           "static_scratch.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"--offload-arch={ARCH}",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc", "-munsafe-fp-atomics"]


# Per-source extra flags.  The matrix-core decode kernels rescale their MFMA
# accumulators with vector instructions, so they keep them in VGPRs rather than
# copying them between AGPRs and VGPRs on every rescale.
EXTRA = {"decode_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "decode_mfma_append.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "decode_mfma_heads.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "decode_mfma_heads_append.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "decode_mfma_multi.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "cascade.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src),
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    # the host pass does not know the gfx950 feature flag; that warning is expected
    warn = "\n".join(x for x in res.stderr.splitlines() if "packed-fp32-ops" not in x).strip()
    if warn and verbose:
        print(warn, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
