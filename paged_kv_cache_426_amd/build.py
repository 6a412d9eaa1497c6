"""Build libpa.so (the C ABI plus the gfx950 kernels) in-tree with hipcc.

    python -m paged_kv_cache_426_amd.build [--verbose]

Every call compiles from source (no caching), writing
``paged_kv_cache_426_amd/libpa.so`` atomically.
"""

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpa.so")

SOURCES = ["pa_api.cpp", "pa_decode.hip", "pa_cache.hip"]

ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the fp8 slot write divides by the scale: IEEE float32 division
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: libpa.so cannot be built")


def build(verbose: bool = False, extra_flags=()) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    fd, tmp = tempfile.mkstemp(prefix=".libpa.", suffix=".so.tmp", dir=PKG)
    os.close(fd)
    cmd = [hipcc(), *FLAGS, *extra_flags, f"-I{INCLUDE}", f"-I{CSRC}", *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        os.unlink(tmp)
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
