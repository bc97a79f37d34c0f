"""Builds libgdn.so (HIP kernels for gfx950 + the C-ABI) in this directory.

    python -m gated_delta_rule_linear_amd.build

Every HIP translation unit is compiled with hipcc for gfx950 only and with
packed-fp32 instruction selection turned off; the host part of the build does
not know that feature and says so once per file, which is harmless.
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libgdn.so")
SOURCES = ["gdn_api.cpp", "gdn_api_backward.cpp", "gdn_api_tiles.cpp", "gdn_prefill.hip", "gdn_decode.hip",
           "gdn_backward.hip", "gdn_tiles.hip", "gdn_noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", f"-I{INCLUDE}", f"-I{CSRC}"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


# The host-sanitizer build (libgdn_hostsan.so): the host code compiled with
# AddressSanitizer and UndefinedBehaviorSanitizer (the kernels are not), for the
# CPU test tier under tests/run_host_sanitizers.sh.
LIB_HOSTSAN = os.path.join(HERE, "libgdn_hostsan.so")
HOSTSAN_FLAGS = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def build(verbose: bool = False, host_sanitize: bool = False) -> str:
    """Compile every source and link libgdn.so (host_sanitize: libgdn_hostsan.so);
    returns its path."""
    lib = LIB_HOSTSAN if host_sanitize else LIB
    extra = HOSTSAN_FLAGS if host_sanitize else []
    with tempfile.TemporaryDirectory(prefix="gdn_build_") as tmp:
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            out = _run([HIPCC, *FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
            if verbose and out.strip():
                print(out)
            objs.append(obj)
        tmp_lib = lib + f".tmp{os.getpid()}"
        link = ["-Xarch_host", "-fsanitize=address,undefined", "-shared-libsan"] if host_sanitize else []
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link, "-o", tmp_lib, *objs])
        os.replace(tmp_lib, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, host_sanitize="--host-sanitize" in sys.argv))
