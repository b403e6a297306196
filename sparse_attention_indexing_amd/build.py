"""Build the HIP shared libraries in-tree for gfx950.

  liblsa.so        the C-ABI library (include/lsa.h): host orchestration + kernels
  liblsa_synth.so  the harness-only synthetic-input generator (lsa_synth)

Run ``python -m sparse_attention_indexing_amd.build`` (or
``__graft_entry__.build()``).  Objects are compiled in parallel into
``_build/`` and linked with hipcc.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
DEVICE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep fp32 arithmetic out of packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

LIB_SOURCES = ["lsa_api.cpp", "lsa_build.hip", "lsa_index.hip", "lsa_attn.hip", "lsa_dense.hip"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build failed: " + " ".join(cmd))
    return r


def _compile(src: str, obj: str, extra=()):
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    _run([HIPCC, *DEVICE_FLAGS, *lang, *extra, "-I", os.path.join(ROOT, "include"),
          "-c", src, "-o", obj])
    return obj


def build(verbose: bool = True) -> list[str]:
    """Compile and link both libraries.  Builds hold an exclusive lock on
    _build/.lock, so two builds started together run one after the other
    instead of writing the same objects at once."""
    import fcntl
    os.makedirs(BUILD, exist_ok=True)
    with open(os.path.join(BUILD, ".lock"), "w") as lock:
        fcntl.flock(lock, fcntl.LOCK_EX)
        return _build(verbose)


def _build(verbose: bool) -> list[str]:
    jobs = []
    for s in LIB_SOURCES:
        jobs.append((os.path.join(CSRC, s), os.path.join(BUILD, s + ".o")))
    synth_src = os.path.join(ROOT, "lsa_synth", "csrc", "synth.hip")
    synth_obj = os.path.join(BUILD, "synth.hip.o")
    jobs.append((synth_src, synth_obj))
    workers = min(len(jobs), int(os.environ.get("MAX_JOBS", "8")))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    lib = os.path.join(PKG, "liblsa.so")
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", lib + ".tmp",
          *objs[:len(LIB_SOURCES)]])
    os.replace(lib + ".tmp", lib)
    synth_lib = os.path.join(ROOT, "lsa_synth", "liblsa_synth.so")
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", synth_lib + ".tmp", synth_obj])
    os.replace(synth_lib + ".tmp", synth_lib)
    if verbose:
        print(f"built {lib}\nbuilt {synth_lib}")
    return [lib, synth_lib]


if __name__ == "__main__":
    build()
