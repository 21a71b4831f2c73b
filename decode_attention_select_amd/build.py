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
    # keep MFMA accumulators in ordinary VGPRs (no AGPR copies around VALU use;
    # a loop of MFMA and independent VALU also ran about 10 % faster in this
    # form than with AGPR accumulators)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# (source, extra flags): decode.hip is compiled twice, one half of its kernel
# variants each, so that the two halves build in parallel
UNITS = [("api.hip", []), ("select.hip", []), ("quant.hip", []), ("ceiling.hip", []),
         ("decode.hip", ["-DKVQ_DECODE_PART=0"]), ("decode.hip", ["-DKVQ_DECODE_PART=1"])]


STAMPS_LIB = os.path.join(PKG, "libkvq_stamps.so")
# per-kernel registers, scratch and spills of libkvq.so, from the compiler's
# resource-usage remarks (written by build(); not part of the library)
RESOURCES = os.path.join(PKG, "kernel_resources.txt")


def _resource_rows(text: str) -> list[tuple[str, dict]]:
    """(kernel, {field: value}) from -Rpass-analysis=kernel-resource-usage
    remarks, in the order the compiler printed them."""
    rows: list[tuple[str, dict]] = []
    for line in text.splitlines():
        if "remark:" not in line or "kernel-resource-usage" not in line:
            continue
        body = line.split("remark:", 1)[1].rsplit("[-Rpass", 1)[0].strip()
        key, _, val = body.partition(":")
        if key == "Function Name":
            rows.append((val.strip(), {}))
        elif rows:
            rows[-1][1][key.strip()] = val.strip()
    return rows


REPORT_KEYS = ("VGPRs", "AGPRs", "TotalSGPRs", "ScratchSize [bytes/lane]", "VGPRs Spill",
               "SGPRs Spill", "LDS Size [bytes/block]", "Occupancy [waves/SIMD]")


def write_resources(rows: list[tuple[str, dict]], path: str = RESOURCES) -> None:
    with open(path, "w") as f:
        f.write("# kernel | " + " | ".join(REPORT_KEYS) + "\n")
        for name, r in rows:
            f.write(" | ".join([name] + [r.get(k, "?") for k in REPORT_KEYS]) + "\n")


def read_resources(path: str = RESOURCES) -> list[tuple[str, dict]]:
    rows = []
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        cols = [c.strip() for c in line.split(" | ")]
        rows.append((cols[0], dict(zip(REPORT_KEYS, cols[1:]))))
    return rows


def check_resources(rows: list[tuple[str, dict]]) -> list[str]:
    """Kernels that use scratch memory or spill vector registers: every
    kernel of the library keeps its state in registers and LDS (scalar
    spills land in vector-register lanes, no memory, and are allowed)."""
    return [name for name, f in rows
            if any(int(f.get(k, "0")) for k in ("ScratchSize [bytes/lane]", "VGPRs Spill"))]


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
            remarks = [] if vflags else ["-Rpass-analysis=kernel-resource-usage"]
            cmd = [HIPCC] + [f for f in FLAGS if f != "-shared"] + vflags + extra + remarks + \
                  ["-c", "-o", obj, os.path.join(CSRC, src)]
            if verbose:
                print(" ".join(cmd), flush=True)
            objs[lib].append(obj)
            err = open(obj + ".err", "w+")
            procs.append((subprocess.Popen(cmd, stderr=err), err))
    try:
        failed, text = [], []
        for p, err in procs:
            failed.append(p.wait())
            err.seek(0)
            out = err.read()
            err.close()
            os.remove(err.name)
            text.append(out)
            # compiler diagnostics other than the resource remarks pass through
            rest = [ln for ln in out.splitlines() if "kernel-resource-usage" not in ln
                    and not ln.lstrip().startswith(("|", "^")) and not ln[:6].strip().isdigit()]
            if rest:
                print("\n".join(rest), file=sys.stderr, flush=True)
        if any(failed):
            raise subprocess.CalledProcessError(max(failed), "hipcc")
        rows = _resource_rows("\n".join(text))
        write_resources(rows)
        bad = check_resources(rows)
        if bad:
            raise RuntimeError("kernels with scratch memory or vector spills (%s): %s"
                               % (RESOURCES, ", ".join(bad)))
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
