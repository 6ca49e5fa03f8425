"""Builds the native libraries in-tree.

  libspa.so              - the product: HIP kernels for gfx950 + the C ABI (include/spa.h)
  synth/libspa_synth_host.so - seeded input generator, host side (gcc + OpenMP)
  synth/libspa_synth_dev.so  - seeded input generator, device side (HIP)

Run `python -m spatially_pipelined_attention_amd.build`.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SYNTH = os.path.join(PKG, "synth")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libspa.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 ALU ops are kept out of generated code.
HIP_CFLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Wno-unused-result", "-munsafe-fp-atomics"]
HIP_FLAGS = HIP_CFLAGS + ["-shared"]
OBJ = os.path.join(ROOT, "_build")


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def _atomic_out(path):
    return path + ".tmp"


def build_synth():
    host_out = os.path.join(SYNTH, "libspa_synth_host.so")
    _run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
          os.path.join(SYNTH, "gen_host.c"), "-o", _atomic_out(host_out), "-lm"])
    os.replace(_atomic_out(host_out), host_out)
    dev_out = os.path.join(SYNTH, "libspa_synth_dev.so")
    _run([HIPCC] + HIP_FLAGS + [os.path.join(SYNTH, "gen_dev.hip"), "-o", _atomic_out(dev_out)])
    os.replace(_atomic_out(dev_out), dev_out)


def product_sources():
    srcs = []
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".cpp")):
            srcs.append(os.path.join(CSRC, name))
    return srcs


def build_product():
    """Every translation unit compiled on its own (in parallel), then linked."""
    srcs = product_sources()
    if not srcs:
        return
    os.makedirs(OBJ, exist_ok=True)
    objs = [os.path.join(OBJ, os.path.basename(s) + ".o") for s in srcs]
    jobs = max(1, min(len(srcs), os.cpu_count() or 1, 16))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        futs = [ex.submit(_run, [HIPCC] + HIP_CFLAGS + ["-I", INCLUDE, "-I", CSRC, "-c", s, "-o", o])
                for s, o in zip(srcs, objs)]
        for f in futs:
            f.result()
    _run([HIPCC] + HIP_FLAGS + objs + ["-o", _atomic_out(LIB), "-lpthread"])
    os.replace(_atomic_out(LIB), LIB)


def build_all():
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    build_synth()
    build_product()


if __name__ == "__main__":
    build_all()
    sys.exit(0)
