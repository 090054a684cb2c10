"""Build libattn.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m transformer_attn_bwd_amd.build   (or call build()).
The library is written next to this file so that it travels with the tree.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

try:
    from .hazards import check_asm
except ImportError:            # run as a script
    from hazards import check_asm

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libattn.so")
OBJ_DIR = os.path.join(ROOT, "_build")

# (source, element type or None): the MFMA kernel files are compiled once per
# 16-bit element type, so that the slow instantiations build in parallel.
ELEMS = ("bf16", "f16")
MFMA_SOURCES = ["attn_fwd_mfma.hip", "attn_bwd_mfma.hip", "attn_bwd_dkdv_dqa.hip",
                "attn_bwd_dkdv_dss.hip", "attn_bwd_dq_mfma.hip", "attn_bwd_dq_ds.hip",
                "attn_proj_gemm.hip"]
SOURCES = ["attn_api.hip", "attn_f32.hip", *MFMA_SOURCES]
UNITS = [("attn_api.hip", None), ("attn_f32.hip", None)] + [
    (src, elem) for src in MFMA_SOURCES for elem in ELEMS]
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-I", INCLUDE, "-I", CSRC,
    # keep hipcc from forming packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results and accumulators in architectural VGPRs: the kernels need
    # their softmax inputs in VGPRs anyway, and this avoids AGPR copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _compile(unit: tuple[str, str | None], extra: list[str]) -> tuple[str, list[str]]:
    """Compile one unit; returns the object and the hazard-check findings
    in its device assembly (kept, with -save-temps, in a directory of its
    own under _build)."""
    src, elem = unit
    stem = os.path.splitext(src)[0] + (f"_{elem}" if elem else "")
    obj = os.path.join(OBJ_DIR, stem + ".o")
    temps = os.path.join(OBJ_DIR, stem)
    os.makedirs(temps, exist_ok=True)
    defs = [f"-DATTN_ELEM={elem}"] if elem else []
    cmd = [hipcc(), *COMMON_FLAGS, *defs, *extra, "-save-temps", "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=temps)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    findings = []
    for asm in glob.glob(os.path.join(temps, f"*-hip-amdgcn-amd-amdhsa-{ARCH}.s")):
        with open(asm) as f:
            findings += [f"{os.path.relpath(asm, ROOT)}: {v}" for v in check_asm(f.read())]
    for big in glob.glob(os.path.join(temps, "*.hipi")) + glob.glob(os.path.join(temps, "*.bc")):
        os.remove(big)
    return obj, findings


def build(extra_flags: list[str] | None = None, verbose: bool = False) -> str:
    """Compile every source and link libattn.so; returns its path."""
    extra = list(extra_flags or [])
    os.makedirs(OBJ_DIR, exist_ok=True)
    workers = max(1, min(len(UNITS), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        done = list(ex.map(lambda u: _compile(u, extra), UNITS))
    objs = [o for o, _ in done]
    findings = [v for _, f in done for v in f]
    if findings:
        raise RuntimeError("AGPR accumulator read or written too soon after an inline-asm MFMA "
                           "(see transformer_attn_bwd_amd/hazards.py):\n" + "\n".join(findings[:20]))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(extra_flags=sys.argv[1:], verbose=True)
