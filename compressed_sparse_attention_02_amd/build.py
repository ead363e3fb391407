"""Build libcsa2.so (HIP, gfx950) in place with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcsa2.so")
SOURCES = ["abi.hip", "index.hip", "index_mx.hip", "topk.hip", "reindex.hip", "attend.hip", "kvwrite.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Werror", "-Wno-unused-command-line-argument",
    # no packed fp32 (v_pk_*_f32) instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer (the argument checks and launch code of
# every entry point; device code is built as usual), for CPU test runs with clang's runtime
# preloaded.  Each sanitizer flag applies to the host compilation only.
LIB_SAN = os.path.join(HERE, "libcsa2_san.so")
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g0"]


def build(verbose: bool = False, extra=(), sanitize: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out = LIB_SAN if sanitize else LIB
    san = HOST_SANITIZE if sanitize else []
    cmd = [hipcc, *FLAGS, *san, *extra, *[os.path.join(CSRC, s) for s in SOURCES], "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
