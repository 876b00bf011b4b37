"""Build the HIP library ``libmoe_mxfp4.so`` in-tree for gfx950.

``python -m mxfp4_mixture_experts_router_amd.build`` (or ``build()``) compiles
every HIP source under ``csrc/`` with hipcc into one shared library beside this
file, and writes a small manifest (version, arch, sha256 of each source and of
the library) next to it.
"""

from __future__ import annotations

import hashlib
import json
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmoe_mxfp4.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["plan.hip", "expert_kernels.hip", "down4_kernel.hip", "scaled_kernels.hip", "stream_kernel.hip",
           "token_down_kernel.hip", "moe_mxfp4_api.hip"]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _sha256(path: str) -> str:
    h = hashlib.sha256()
    with open(path, "rb") as f:
        for chunk in iter(lambda: f.read(1 << 20), b""):
            h.update(chunk)
    return h.hexdigest()


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, LIB_PATH)
    manifest = {
        "library": LIB_NAME,
        "arch": ARCH,
        "flags": HIPCC_FLAGS,
        "sources": {s: _sha256(os.path.join(CSRC, s)) for s in SOURCES},
        "headers": {h: _sha256(os.path.join(d, h)) for d, h in
                    ((INCLUDE, "moe_mxfp4.h"), (CSRC, "kernels.h"), (CSRC, "device_common.h"), (CSRC, "list_common.h"),
                     (CSRC, "route_plan.h"))},
        "library_sha256": _sha256(LIB_PATH),
    }
    with open(os.path.join(PKG_DIR, "libmoe_mxfp4.manifest.json"), "w") as f:
        json.dump(manifest, f, indent=1)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
