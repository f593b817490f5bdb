"""Build libvimscan.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "vimscan.hip")
SRCS = [SRC, os.path.join(PKG, "csrc", "proj.hip"), os.path.join(PKG, "csrc", "host.cpp")]
LIB = os.path.join(PKG, "libvimscan.so")
INCLUDE = os.path.join(ROOT, "include")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
    # packed-fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def scratch_kernels(log: str):
    """Kernels whose resource-usage remark reports scratch memory: register
    arrays that did not stay in registers (a step left out of line, a
    dynamic index), which costs an order of magnitude in time."""
    bad, name = [], None
    for line in log.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            bad.append((name, int(m.group(1))))
    return bad


def build(out: str = LIB, extra=()) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-Rpass-analysis=kernel-resource-usage", *extra, "-I", INCLUDE,
           *SRCS, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building %s" % out)
    bad = scratch_kernels(r.stderr)
    if bad:
        os.remove(tmp)
        raise RuntimeError("kernels use scratch memory: " +
                           ", ".join("%s (%d B/lane)" % b for b in bad))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
