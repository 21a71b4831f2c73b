"""Builds libkvq.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkvq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # fp32 division and sqrt correctly rounded (the quantizer and the pair
    # norms are bit-exact IEEE computations)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in ordinary VGPRs (no AGPR copies around VALU use)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# (source, extra flags): decode.hip is compiled twice, one half of its kernel
# variants each, so that the two halves build in parallel
UNITS = [("api.hip", []), ("select.hip", []), ("quant.hip", []), ("ceiling.hip", []),
         ("decode.hip", ["-DKVQ_DECODE_PART=0"]), ("decode.hip", ["-DKVQ_DECODE_PART=1"])]


STAMPS_LIB = os.path.join(PKG, "libkvq_stamps.so")


def build(verbose: bool = False, stamps: bool = True) -> str:
    """Compiles every unit to an object (in parallel), then links libkvq.so.
    With `stamps`, also libkvq_stamps.so: the same sources with the decode
    kernel's phase timestamps compiled in (-DKVQ_STAMPS; measurement only)."""
    tag = "%d" % os.getpid()
    variants = [(LIB, [])] + ([(STAMPS_LIB, ["-DKVQ_STAMPS"])] if stamps else [])
    objs, procs = {}, []
    for lib, vflags in variants:
        objs[lib] = []
        for i, (src, extra) in enumerate(UNITS):
            obj = os.path.join(PKG, "_unit%d%s.%s.o" % (i, "s" if vflags else "", tag))
            cmd = [HIPCC] + [f for f in FLAGS if f != "-shared"] + vflags + extra + \
                  ["-c", "-o", obj, os.path.join(CSRC, src)]
            if verbose:
                print(" ".join(cmd), flush=True)
            objs[lib].append(obj)
            procs.append(subprocess.Popen(cmd))
    try:
        failed = [p.wait() for p in procs]
        if any(failed):
            raise subprocess.CalledProcessError(max(failed), "hipcc")
        for lib, _ in variants:
            tmp = lib + ".tmp" + tag
            cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs[lib]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.check_call(cmd)
            os.replace(tmp, lib)
    finally:
        for ol in objs.values():
            for o in ol:
                if os.path.exists(o):
                    os.remove(o)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
