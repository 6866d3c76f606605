"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code, for the CPU test-suite.

- libdlfusion: every source built for gfx950 as usual, with the sanitizers on the host side only
  (-Xarch_host before each -fsanitize=; device code is never instrumented), so that the C ABI's
  validation, the BN fold, the fusion pass and the FFN packing run instrumented on the CPU.
- liboracle: oracle.c built with clang and the same sanitizers (the runtime must be the one the
  library uses).

Both go to dl_fusion_amd/_build_san/ and are rebuilt only when their sources change.  The test
that uses them (test_sanitizers.py) preloads clang's ASan runtime into a child Python process and
points the binding and the oracle at these builds (DLF_LIBRARY, ORACLE_LIBRARY).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import hashlib
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dl_fusion_amd", "csrc")
OUT = os.path.join(ROOT, "dl_fusion_amd", "_build_san")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _hash(paths, extra: str) -> str:
    h = hashlib.sha256(extra.encode())
    for p in sorted(paths):
        with open(p, "rb") as f:
            h.update(p.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def _stamp_ok(path: str, digest: str) -> bool:
    try:
        with open(path + ".hash") as f:
            return f.read().strip() == digest and os.path.exists(path)
    except OSError:
        return False


def build_library() -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    hdrs = glob.glob(os.path.join(CSRC, "*.h")) + [os.path.join(ROOT, "include", "dlfusion.h")]
    lib = os.path.join(OUT, "libdlfusion_san.so")
    digest = _hash(srcs + hdrs, " ".join(HOST_SAN))
    if _stamp_ok(lib, digest):
        return lib
    os.makedirs(OUT, exist_ok=True)

    def one(src):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"), *HOST_SAN, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitizer build of {src} failed:\n{r.stderr[-3000:]}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(one, srcs))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-shared-libsan", "-o", lib, *objs]
    subprocess.run(cmd, check=True, capture_output=True)
    with open(lib + ".hash", "w") as f:
        f.write(digest)
    return lib


def build_oracle() -> str:
    src = os.path.join(ROOT, "oracle", "oracle.c")
    lib = os.path.join(OUT, "liboracle_san.so")
    flags = ["-std=c11", "-O1", "-g", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
             "-D_GNU_SOURCE", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-shared-libsan"]
    digest = _hash([src], " ".join(flags))
    if _stamp_ok(lib, digest):
        return lib
    os.makedirs(OUT, exist_ok=True)
    subprocess.run([CLANG, *flags, "-o", lib, src, "-lm"], check=True, capture_output=True)
    with open(lib + ".hash", "w") as f:
        f.write(digest)
    return lib
