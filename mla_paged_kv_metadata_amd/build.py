"""Build the gfx950 HIP library libmla_decode.so in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmla_decode.so")
SOURCES = ["mla_api.cpp", "mla_metadata.hip", "mla_decode.hip"]

# Packed fp32 VALU forms are disabled for all device code (hipcc's host pass
# warns that it does not know the feature; that warning is harmless).
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


# The race-check variant: every page copy issued only after the workgroup is
# done with the page before it (MLA_SERIAL_COPIES in csrc/mla_decode.hip);
# its results must equal the default library's bit for bit.
SERIAL_LIB = os.path.join(PKG, "libmla_decode_serial.so")
VARIANTS = {LIB: [], SERIAL_LIB: ["-DMLA_SERIAL_COPIES=1"]}


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source into libmla_decode.so and the race-check variant
    libmla_decode_serial.so (always recompiles; the two compile in parallel)."""
    procs = []
    for lib, flags in VARIANTS.items():
        tmp = lib + ".tmp"
        cmd = [hipcc(), *HIPCC_FLAGS, *flags, *extra_flags, "-I", os.path.join(ROOT, "include"), "-o", tmp,
               *[os.path.join(CSRC, s) for s in SOURCES]]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((lib, tmp, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    noise = "is not a recognized feature for this target"
    failed = []
    for lib, tmp, pr in procs:
        outp, _ = pr.communicate()
        err = "\n".join(l for l in outp.splitlines() if noise not in l)
        if pr.returncode != 0:
            failed.append(f"{os.path.basename(lib)}: hipcc failed ({pr.returncode}):\n{err}")
            continue
        if verbose and err.strip():
            print(err, file=sys.stderr)
        os.replace(tmp, lib)
    if failed:
        raise RuntimeError("\n".join(failed))
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
