"""Build step of the HIP library: compiles csrc/*.hip for gfx950 into libgrok_moe.so (in-tree)."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libgrok_moe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU instructions stay off in every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def scratch_kernels(remarks: str):
    """Kernels whose resource-usage remark reports private (scratch) memory:
    a register array the compiler could not keep in registers, which costs a
    memory round trip per access in the hot loops."""
    bad, name = [], None
    for line in remarks.splitlines():
        if "Function Name:" in line:
            name = line.split("Function Name:", 1)[1].split("[")[0].strip()
        elif "ScratchSize [bytes/lane]:" in line and name:
            size = int(line.split("ScratchSize [bytes/lane]:", 1)[1].split("[")[0].strip())
            if size:
                bad.append((name, size))
    return bad


def build(verbose: bool = False) -> str:
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-Rpass-analysis=kernel-resource-usage"] + inc + sources() + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    lines = (res.stderr or "").splitlines()
    err = "\n".join(l for l in lines if noise not in l and "remark:" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    bad = scratch_kernels(res.stderr or "")
    if bad:
        os.remove(tmp)
        raise RuntimeError("kernels use scratch memory: " + ", ".join(f"{n} ({b} B/lane)" for n, b in bad))
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
