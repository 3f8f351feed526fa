"""Build ``libqpack.so`` (gfx950) in-tree with hipcc.

Run as ``python conv_qpack_weights_amd/build.py`` (a plain script: importing
the package needs the library); ``__graft_entry__.build()`` calls :func:`build`.
Every HIP source is compiled for gfx950 only, with packed-FP32 instruction
selection disabled and FP contraction handled per file (the numeric kernels
turn it off).  The link refuses undefined symbols, so a kernel whose host
stub was not emitted fails here rather than at load time.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqpack.so")
# Measurement-only kernels (read-only HBM stream, int8 MFMA loop): a library
# of their own, loaded by the benchmark only.
FLOORS_SRC = "floors.hip"
FLOORS_LIB = os.path.join(HERE, "libqpfloors.so")
SOURCES = ["status.cpp", "pack.hip", "quant.hip", "im2col.hip", "gemm_s8.hip", "conv.hip",
           "conv_implicit.hip", "a8w4.hip", "a8w8b.hip", "unpack.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fno-gpu-rdc", "-Wall", "-Wno-unused-result", "-Wno-unused-variable"]


# Per-file code-generation options.  The A8W4 kernels rescale every MFMA
# result on the VALU right away, and the implicit-GEMM convolution keeps
# few accumulators, so their MFMAs write VGPRs (no AGPR copies).
EXTRA = {"a8w4.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
         "conv_implicit.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]}


def _compile(src: str, obj: str) -> None:
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    subprocess.check_call(cmd)


def build(verbose: bool = True, jobs: int = 4) -> str:
    from concurrent.futures import ThreadPoolExecutor

    with tempfile.TemporaryDirectory(prefix="qpack_build_") as tmp:
        objs = [os.path.join(tmp, s + ".o") for s in SOURCES]
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            list(ex.map(lambda so: _compile(*so), zip(SOURCES, objs)))
        out_tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs,
                               "-o", out_tmp, "-Wl,--no-undefined", "-lamdhip64"])
        os.replace(out_tmp, LIB)
        fobj = os.path.join(tmp, FLOORS_SRC + ".o")
        _compile(FLOORS_SRC, fobj)
        ftmp = FLOORS_LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", fobj, "-o",
                               ftmp, "-Wl,--no-undefined", "-lamdhip64"])
        os.replace(ftmp, FLOORS_LIB)
    if verbose:
        print("built", LIB, "and", FLOORS_LIB)
    return LIB


if __name__ == "__main__":
    build(jobs=int(sys.argv[1]) if len(sys.argv) > 1 else 4)
