"""Build the gfx950 library ``libpkv.so`` in-tree with hipcc.

Usage: ``python -m paged_kv_gqa_pkv_amd.build`` (or ``build()`` from Python).
Always recompiles.  Objects go to ``_build/`` (one hipcc per source, run in
parallel), the shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libpkv.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

SOURCES = ["kv_append.hip", "decode.hip", "prefill.hip", "mixed.hip", "qk_rope.hip", "pkv_api.cpp"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep packed-fp32 instructions out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


# Per-source extra flags.  prefill.hip, mixed.hip (which holds the prefill
# kernel's body too): keep the MFMA accumulators in VGPRs
# (otherwise, with more than 256 registers, they land in AGPRs and every
# tile copies them back and forth for the softmax rescale).
EXTRA = {
    "prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "mixed.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _compile(hipcc: str, src: str, verbose: bool, defines, build_dir: str) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc, *COMMON, *EXTRA.get(src, []), *[f"-D{d}" for d in defines], "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(verbose: bool = False, defines=(), out: str = OUT) -> str:
    """Compile every source and link ``out``.  ``defines`` (NAME=VALUE strings)
    override the kernels' tuning constants."""
    build_dir = BUILD_DIR if out == OUT else os.path.join(
        BUILD_DIR, os.path.splitext(os.path.basename(out))[0])
    os.makedirs(build_dir, exist_ok=True)
    hipcc = _hipcc()
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s, verbose, defines, build_dir), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
