"""Build the HIP libraries for gfx950, in-tree: ``libreplayssm.so`` (the
decode path's C ABI, include/replayssm.h) and ``librssm_probes.so`` (the HBM
probes that measure the device's ceilings, include/rssm_probes.h).

Each source compiles separately (in parallel) to an object under ``_build/``,
then hipcc links each shared library next to this file.  All device code is
built with packed fp32 arithmetic disabled (``-packed-fp32-ops``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libreplayssm.so")
SOURCES = ["rssm_kernels.hip", "rssm_decode_split.hip", "rssm_verify.hip", "rssm_prefill.hip", "conv_kernels.hip",
           "replayssm_api.hip"]
PROBE_LIB = os.path.join(HERE, "librssm_probes.so")
PROBE_SOURCES = ["probe_kernels.hip", "probe_api.hip"]
ARCH = os.environ.get("RSSM_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         f"-I{INCLUDE}", f"-I{CSRC}", "-Wno-unused-command-line-argument"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-4000:]}")
    return obj


def _link(lib: str, objs) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(lib)} failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link(LIB, [objs[s] for s in SOURCES])
    _link(PROBE_LIB, [objs[s] for s in PROBE_SOURCES])
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
