"""Build libpiattn.so in-tree with hipcc for gfx950.

    python -m sparse_long_context_piattn_amd.build

Every source under csrc/ is compiled for the MI355X (gfx950) device and the
x86-64 host and linked into sparse_long_context_piattn_amd/libpiattn.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libpiattn.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "neighbors.hip", "fwd_gather.hip", "fwd_resid.hip",
           "fwd_split.hip", "fwd_f32mfma.hip", "decode.hip", "bwd.hip", "bwd_band.hip",
           "proj.hip", "noalloc.hip"]

# Packed-fp32 VALU forms are kept out of the device code (plain fp32 only).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "--offload-arch=" + ARCH, "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    cc = hipcc()
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with tempfile.TemporaryDirectory(prefix="piattn_build_") as tmp:
        procs, objs = [], []
        for s in srcs:
            obj = os.path.join(tmp, s + ".o")
            cmd = [cc, "-c", os.path.join(CSRC, s), "-o", obj] + COMMON
            if s.endswith(".hip"):
                cmd = [cc, "-x", "hip", "-c", os.path.join(CSRC, s), "-o", obj] + COMMON + DEVICE_FLAGS
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                              stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        errors = []
        for s, p in procs:
            out, _ = p.communicate()
            # the host pass does not know the device-only feature flag: not an error
            lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
            if p.returncode != 0:
                errors.append("%s:\n%s" % (s, "\n".join(lines)))
            elif verbose and lines:
                print("\n".join(lines))
        if errors:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
        tmp_lib = os.path.join(tmp, "libpiattn.so")
        cmd = [cc, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp_lib] + objs
        subprocess.check_call(cmd)
        shutil.copyfile(tmp_lib, LIB + ".tmp%d" % os.getpid())
        os.replace(LIB + ".tmp%d" % os.getpid(), LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
