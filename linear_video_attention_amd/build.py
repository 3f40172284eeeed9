"""Build the HIP library ``libvdn.so`` in-tree for gfx950 with hipcc.

Every call recompiles every source (no staleness checks), then links the shared library next to
this file.  Object files go to ``_build/`` beside it.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libvdn.so")

SOURCES = [
    "plan.cpp",
    "abi.cpp",
    "prep_kv.hip",
    "softmax_simt.hip",
    "softmax_mfma.hip",
    "prep_fp8.hip",
    "softmax_fp8.hip",
    "vda.hip",
    "vda_stats_mfma.hip",
    "vda_invert_mfma.hip",
    "vda_scan_mfma.hip",
    "epilogue_simt.hip",
    "epilogue_mfma.hip",
    "calibrate.hip",
    "backward.hip",
    "backward_mfma.hip",
    "merge_bwd_mfma.hip",
    "xty_mfma.hip",
    "scan_bwd_mfma.hip",
    "noalloc.hip",
]

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 instructions are kept out of the generated code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]

# Per-source flags.  The window-softmax kernel is scheduled by LLVM's instruction-level-parallelism
# strategy: its matrix and vector instruction streams interleave better (about 4 % faster at 768p,
# identical results).  The backward softmax transposes use the memory-clause strategy: fewer
# spilled registers in dK/dV and about 4 % less time per backward call at 768p (identical results).
FILE_FLAGS = {
    "softmax_mfma.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
    "backward_mfma.hip": ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, verbose: bool, out_dir: str, extra: list) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-x", "hip", *FLAGS, *FILE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, jobs: int = 8, lib_path: str = LIB_PATH, extra_flags=()) -> str:
    """Compile every source and link ``lib_path`` (default: the in-tree libvdn.so)."""
    out_dir = OUT_DIR if lib_path == LIB_PATH else lib_path + ".objs"
    os.makedirs(out_dir, exist_ok=True)
    extra = list(extra_flags)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, out_dir, extra), SOURCES))
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose=True))
