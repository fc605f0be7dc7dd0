"""Build libqmv.so (the product library) and libqmv_ceilings.so (the
benchmark's measurement kernels) in-tree with hipcc for gfx950.

    python -m gguf_quantized_matvec_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqmv.so")
CEIL_LIB = os.path.join(HERE, "libqmv_ceilings.so")
CEIL_SRC = os.path.join(CSRC, "qmv_ceilings.hip")
# (source, extra flags): the GEMV kernels take MFMA results straight into
# VGPRs (no accumulation-register copies); the GEMM keeps the default choice
SOURCES = [(os.path.join(CSRC, "qmv_kernels.hip"), ["-mllvm", "-amdgpu-mfma-vgpr-form"]),
           (os.path.join(CSRC, "qmm_kernels.hip"), []),
           (os.path.join(CSRC, "qmm8k_kernels.hip"), []),
           (os.path.join(CSRC, "qmv_noalloc.hip"), []),
           (os.path.join(CSRC, "qmv_api.cpp"), [])]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # exact f32 arithmetic: no contraction of a*b+c, correctly rounded divide
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed-fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _run(cmd: list) -> None:
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libqmv.so")


def build() -> str:
    # the translation units compile in parallel (one hipcc process each)
    from concurrent.futures import ThreadPoolExecutor
    srcs = SOURCES + [(CEIL_SRC, [])]
    objs = [os.path.join(CSRC, os.path.basename(src) + ".o") for src, _ in srcs]
    with ThreadPoolExecutor(len(srcs)) as ex:
        for f in [ex.submit(_run, [HIPCC, *FLAGS, *extra, "-x", "hip", "-c", src, "-o", obj])
                  for (src, extra), obj in zip(srcs, objs)]:
            f.result()
    for lib, parts in ((LIB, objs[:-1]), (CEIL_LIB, objs[-1:])):
        tmp = lib + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", *parts, "-o", tmp])
        os.replace(tmp, lib)
    for obj in objs:
        os.remove(obj)
    return LIB


if __name__ == "__main__":
    print(build())
