"""Build the gfx950 HIP library libwd.so in-tree with hipcc.

    python -m moe_decode_gate_amd.build        (or build() from Python)

The library is written to moe_decode_gate_amd/lib/libwd.so, next to the
binding that loads it.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
# one translation unit per kernel family, compiled in parallel and linked into one library
SRCS = [os.path.join(PKG, "csrc", f) for f in ("wd.hip", "ec.hip")]
DEPS = SRCS + [os.path.join(PKG, "csrc", f) for f in ("wd_device.h", "wd_kernels.h")] + \
       [os.path.join(ROOT, "include", f) for f in ("wd.h", "ec.h")]
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "libwd.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-FP32 VALU forms in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernel arguments ahead of any aggregate go to SGPRs at dispatch (gfx950 kernarg preload)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


def _finish(proc) -> str:
    _, stderr = proc.communicate()
    err = "\n".join(l for l in stderr.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{err}")
    return err


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    objs = [os.path.join(LIB_DIR, os.path.basename(src)[:-4] + ".o") for src in SRCS]
    procs = [_run([hipcc(), *HIPCC_FLAGS, *extra, *inc, "-c", src, "-o", obj], verbose)
             for src, obj in zip(SRCS, objs)]
    errs = [_finish(p) for p in procs]
    tmp = LIB + ".tmp"
    errs.append(_finish(_run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)))
    err = "\n".join(e for e in errs if e.strip())
    if verbose and err:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
