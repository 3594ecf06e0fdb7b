"""Build libkq.so for gfx950 in-tree: ``python -m post_quantization_04_amd.build``.

Each HIP source is compiled to an object under ``_build/`` (in parallel) and
linked into ``post_quantization_04_amd/libkq.so`` with hipcc. The peak probes
(``csrc/peaks.hip``, not part of the quantization path) go into
``post_quantization_04_amd/libkq_peaks.so``. Packed float32 instructions are
disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libkq.so")
PEAKS_LIB = os.path.join(HERE, "libkq_peaks.so")
SOURCES = ["kq_api.hip", "timing.hip", "syrk.hip", "score.hip", "biip.hip", "chol.hip", "obs.hip",
           "decode.hip", "loss.hip", "gptaq.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libkq")


def flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
    ]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{errs}")
    if errs.strip():
        sys.stderr.write(errs + "\n")
    return obj


def _link(objs: list, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(out)} failed:\n{res.stderr}")
    os.replace(tmp, out)


def build(jobs: int = 8) -> str:
    """Compile every HIP source and link libkq.so and libkq_peaks.so. Returns libkq.so's path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + ["peaks.hip"]
    with concurrent.futures.ThreadPoolExecutor(max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:-1], LIB)
    _link(objs[-1:], PEAKS_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
