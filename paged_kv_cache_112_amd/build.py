"""Compile the HIP sources into the in-tree shared library ``libpa.so`` (gfx950).

Every call recompiles.  Objects go to ``_build/`` next to the sources; the
library lands beside this file, where the Python binding loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB_NAME = "libpa.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
# the checked build: kernels bounds-check slots, block ids and lengths (-DPA_CHECKED=1)
CHECKED_LIB_PATH = os.path.join(HERE, "libpa_checked.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "check.cpp", "write_kv.hip", "copy_blocks.hip", "attention_mfma.hip", "attention_lds.hip", "step_tensors.hip", "decode_mfma.hip", "decode_valu.hip", "merge.hip", "noalloc.hip", "checked.hip"]

# Packed-fp32 instructions are disabled on purpose; fp32 denormals are kept.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"),
]

# Per-source additions.  The multi-query attention kernel keeps its matrix-core
# accumulators in ordinary VGPRs: its rare rescale multiplies them on the vector unit,
# and with accumulation registers the compiler copies every accumulator between the two
# register files at each loop iteration.
SOURCE_FLAGS = {
    "attention_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "attention_lds.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(args):
    cmd, src = args
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return r.stderr


def build(verbose: bool = False, extra_flags: list[str] | None = None, out_path: str | None = None,
          checked: bool = False) -> str:
    """Compile every source for gfx950 and link ``libpa.so`` (``libpa_checked.so`` with
    ``checked``, or ``out_path``); returns its path."""
    cc = hipcc()
    lib_path = out_path or (CHECKED_LIB_PATH if checked else LIB_PATH)
    if checked:
        extra_flags = list(extra_flags or []) + ["-DPA_CHECKED=1"]
    obj_dir = (os.path.join(HERE, "_build_checked" if checked else "_build") if out_path is None
               else lib_path + ".objs")
    os.makedirs(obj_dir, exist_ok=True)
    flags = COMMON_FLAGS + list(extra_flags or [])
    jobs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        jobs.append(([cc, *flags, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj], src))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "8"))))
    with ThreadPoolExecutor(workers) as ex:
        for log in ex.map(_compile, jobs):
            if verbose and log.strip():
                print(log)
    tmp = lib_path + ".tmp"
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose=True))
    print(build(verbose=True, checked=True))
