"""Build libuno.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libuno.so")
SOURCES = ["uno_api.cpp", "uno_noalloc.cpp", "filter_kernels.hip", "sample_kernels.hip", "attention_kernels.hip", "probe_kernels.hip"]
HEADERS = ["uno_device.h", "uno_internal.h", "exp2_table.inc", os.path.join("..", "..", "include", "uno.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    # no packed fp32 instructions (v_pk_*_f32): kernels keep to scalar fp32 ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# The host code of the library under AddressSanitizer and UBSan (device code
# unchanged), for checking the C ABI's host logic on the CPU; load it with
# UNO_LIBRARY=<path> and clang's ASan runtime preloaded.
LIB_SAN = os.path.join(HERE, "libuno_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = LIB_SAN if sanitize else LIB
    tmp = out + ".tmp%d" % os.getpid()
    srcs = []
    for s in SOURCES:
        p = os.path.join(CSRC, s)
        srcs += (["-x", "hip", p] if s.endswith(".hip") else ["-x", "hip", p])
    cmd = [HIPCC] + FLAGS + (SAN_FLAGS if sanitize else []) + ["-I", os.path.join(HERE, "..", "include"), "-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed (exit %d)" % res.returncode)
    os.replace(tmp, out)
    return out


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    for s in SOURCES + HEADERS:
        if os.path.getmtime(os.path.join(CSRC, s)) > t:
            return True
    return False


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv[1:]))
