"""Build the host-AddressSanitizer checker of the libspear C ABI.

    python tests/asan/build_asan.py

Compiles the library's sources with AddressSanitizer on their host code
(the device code is built as usual, uninstrumented) into
_build/asan/libspear_hostasan.so, and links tests/asan/abi_check.cpp against
it into _build/asan/abi_check, which carries the sanitizer runtime itself.
A build is skipped when the sources are those of the last one.
"""

from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "quantized_gemm_error_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(ROOT, "_build", "asan")
SOURCES = ("api.hip", "pack.hip", "decode.hip", "decode_w8.hip", "decode_w4.hip", "wide.hip",
           "prefill.hip")
CHECK = os.path.join(OUT, "abi_check")


def _tool(name: str, fallback: str) -> str:
    path = shutil.which(name) or fallback
    if not os.path.exists(path):
        raise RuntimeError(f"{name} not found")
    return path


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        noise = [ln for ln in res.stderr.splitlines() if "packed-fp32" not in ln]
        raise RuntimeError(" ".join(cmd) + "\n" + "\n".join(noise))


def _sources_hash() -> str:
    h = hashlib.sha256()
    files = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC))
             if f.endswith((".hip", ".h", ".inc"))]
    for path in files + [os.path.join(INCLUDE, "spear.h"), os.path.join(HERE, "abi_check.cpp"),
                         os.path.abspath(__file__)]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def build(force: bool = False) -> str:
    """Build unless the sources are unchanged since the last build; returns the checker's path."""
    stamp = os.path.join(OUT, "sources.sha256")
    digest = _sources_hash()
    if not force and os.path.exists(CHECK) and os.path.exists(stamp):
        with open(stamp) as f:
            if f.read().strip() == digest:
                return CHECK
    hipcc = _tool("hipcc", "/opt/rocm/bin/hipcc")
    clangxx = _tool("amdclang++", "/opt/rocm/lib/llvm/bin/clang++")
    os.makedirs(OUT, exist_ok=True)
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(src):
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        _run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *host_asan,
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    lib = os.path.join(OUT, "libspear_hostasan.so")
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *host_asan, *objs, "-o", lib])
    _run([clangxx, "-std=c++17", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
          "-I", INCLUDE, os.path.join(HERE, "abi_check.cpp"), lib, f"-Wl,-rpath,{OUT}",
          "-o", CHECK])
    with open(stamp, "w") as f:
        f.write(digest + "\n")
    return CHECK


if __name__ == "__main__":
    print(build(force="--force" in sys.argv))
    sys.exit(0)
