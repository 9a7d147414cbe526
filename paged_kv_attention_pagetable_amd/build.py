"""Build the HIP library ``libpkv.so`` in-tree for gfx950.

Every source under ``csrc/`` is compiled with hipcc (device code for gfx950
only) and linked into one shared library next to this file.  Run as
``python -m paged_kv_attention_pagetable_amd.build`` or call ``build()``.
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libpkv.so")
BUILD_DIR = os.path.join(HERE, "_build")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU ops stay off: the compiler must not form v_pk_*_f32.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


# Per-source flags.  The decode kernels take their first four arguments
# (slots, seq_lens, page table, split count), the prefill kernel its first
# five (cu_seqlens, slots, start_pos, page table, sequence count) and the
# prologue kernel its first seven (the same metadata, the raw k and v rows,
# the token count) ahead of their argument structs, so that these arrive
# preloaded in scalar registers and each workgroup's first loads issue
# without waiting for an argument load.
PER_SOURCE = {
    "decode.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=4"],
    "prefill.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=5"],
    "prologue.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=7"],
}


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *PER_SOURCE.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra=None) -> str:
    """Compile and link ``libpkv.so``; returns its path.  Always rebuilds."""
    extra = list(extra or [])
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = min(len(sources), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), sources))
    tmp = OUT + ".tmp"
    # -z defs: an unresolved symbol (e.g. a kernel stub the host pass dropped)
    # fails the link here instead of the first dlopen on a GPU machine.
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Wl,-z,defs", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT} from {len(sources)} sources")
    return OUT


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
