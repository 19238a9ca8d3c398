"""Build libw4a16.so (gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libw4a16.so")
SOURCES = ["w4a16_api.hip", "w4a16_gemm.hip", "w4a16_decode.hip", "w4a16_prefill.hip", "w4a16_aux.hip"]
ARCH = "gfx950"

# -packed-fp32-ops keeps the compiler from forming v_pk_{add,mul,fma}_f32 (the host pass
# warns that it does not know the feature; that is harmless).
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    # keep a one-lane atomic a single atomic whose result is waited for where it is used (the
    # split-K arrival count is read only at the end of the kernel), not a wave-aggregated one
    # waited for on the spot
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    # loop headers on 64-byte instruction-cache lines (the same box, the two builds alternated:
    # FFN down M = 1 / 4 / 8 0.12-0.2 us faster, FFN up M = 2 0.15, no row count slower)
    "-falign-loops=64",
    f"-I{os.path.join(ROOT, 'include')}",
]


def source_hash() -> str:
    """Hash of every HIP source and header the library is built from, and of its compiler flags."""
    import hashlib
    h = hashlib.sha256("\0".join(FLAGS[:-1]).encode())   # the include path (last) depends on the checkout
    names = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h")))
    for n in names + ["../../include/w4a16.h"]:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(n.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile every HIP source into verify_matmul_amd/libw4a16.so (always recompiles)."""
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), *FLAGS, f'-DW4A16_SOURCE_HASH="{source_hash()}"', *[os.path.join(CSRC, s) for s in SOURCES],
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "is not a recognized feature for this target"
    out = "\n".join(l for l in res.stdout.splitlines() if noise not in l)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
