"""Build of libqil with AddressSanitizer and UndefinedBehaviorSanitizer on its
host code (the C ABI's argument checks, split planning and workspace sizing in
api.hip); the device code is compiled as in the regular build.  Used by
tests/test_abi_sanitized.py, which runs the ABI tests against it on the CPU.

Every sanitizer flag goes to the host compiler only (-Xarch_host): the GPU
code objects are the regular ones."""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

from paged_kv_attention_16_amd import build as qbuild  # noqa: E402

OUT = os.path.join(ROOT, "_build", "host_sanitized")
LIB = os.path.join(OUT, "libqil_host_sanitized.so")
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]


def clang():
    return os.path.join(os.path.dirname(os.path.realpath(qbuild.hipcc())), "..", "llvm", "bin", "clang")


def asan_runtime():
    """Path of the ASan runtime shared library of the toolchain's clang."""
    for cand in (os.path.join("/opt/rocm/llvm/bin", "clang"), clang(), shutil.which("clang")):
        if cand and os.path.exists(cand):
            p = subprocess.run([cand, "-print-file-name=libclang_rt.asan-x86_64.so"],
                               capture_output=True, text=True).stdout.strip()
            if p and os.path.exists(p):
                return p
    raise RuntimeError("ASan runtime (libclang_rt.asan-x86_64.so) not found")


def _compile(src):
    obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
    cmd = [qbuild.hipcc(), *qbuild.common_flags(), *qbuild.EXTRA_FLAGS.get(src, []), *SANITIZE,
           "-c", os.path.join(qbuild.CSRC, src), "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{p.stderr}")
    return obj


def build_sanitized():
    os.makedirs(OUT, exist_ok=True)
    with ThreadPoolExecutor(len(qbuild.SOURCES)) as ex:
        objs = list(ex.map(_compile, qbuild.SOURCES))
    cmd = [qbuild.hipcc(), f"--offload-arch={qbuild.ARCH}", "-shared", "-fPIC", *SANITIZE, *objs,
           "-o", LIB]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stderr}")
    return LIB


if __name__ == "__main__":
    print(build_sanitized())
