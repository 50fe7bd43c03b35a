"""Build libtq.so (the HIP library behind include/tq.h) in-tree with hipcc for gfx950.

    python -m dequant_gemv_tq_amd.build_lib            # build
    python -m dequant_gemv_tq_amd.build_lib --asm DIR  # also write device assembly

Every source is compiled on its own (in parallel) into ``_build/`` at the
repository root and linked into ``dequant_gemv_tq_amd/libtq.so``.  Packed
FP32 instructions are disabled for the device pass (the host pass warns that
it does not know the feature; that warning is expected).
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtq.so")
ARCH = "gfx950"

SOURCES = ["tq_api.cpp", "tq_codebook.cpp", "tq_transform.hip", "tq_gemv.hip", "tq_gemm.hip", "tq_blockfp.hip", "tq_kv.hip",
           "tq_q8.hip", "tq_measure.hip"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libtq")
    return path


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc()] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    out = _run(cmd)
    if out.strip():
        print(out)
    return obj


def build(verbose: bool = False, asm_dir: str | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    _run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        for src in SOURCES:
            if src.endswith(".hip"):
                _run([_hipcc()] + FLAGS + ["-S", "--cuda-device-only", os.path.join(CSRC, src), "-o",
                                           os.path.join(asm_dir, os.path.splitext(src)[0] + ".s")])
    if verbose:
        print(f"built {LIB}")
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None)
    a = ap.parse_args(argv)
    build(verbose=True, asm_dir=a.asm)


if __name__ == "__main__":
    sys.exit(main())
