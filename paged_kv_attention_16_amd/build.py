"""Build libqil.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m paged_kv_attention_16_amd.build

Every source under csrc/ is compiled by hipcc in parallel into _build/, then
linked into paged_kv_attention_16_amd/libqil.so (the attention path) and
libqil_ceiling.so (the benchmark's measured-ceiling kernels).  The build always compiles;
it never reuses stale objects.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqil.so")
ARCH = os.environ.get("QIL_OFFLOAD_ARCH", "gfx950")

SOURCES = ["api.hip", "kv_write.hip", "qkv_proj.hip", "decode.hip", "prefill.hip", "mixed.hip",
           "debug_check.hip"]
# measured-ceiling kernels for the benchmark, in a library of their own
CEILING_SOURCE = "ceiling.hip"
CEILING_LIB = os.path.join(PKG, "libqil_ceiling.so")


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libqil)")


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
        "-Wall", "-Wno-unused-function",
        # packed fp32 VALU forms stay off: plain fp32 code only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
    ]


# Per-source extra flags.  prefill.hip: LLVM's max-ILP machine scheduler
# interleaves the tile loop's exponentials and conversions with its MFMAs
# better than the default; measured side by side (same binary otherwise,
# bit-identical outputs): prefill-varlen 121.9 -> 119.5 us, the 8B step's
# prefill 129.6 -> 124.0 us.  mixed.hip (the one-launch step, whose prefill
# tiles run the same tile code): 322 -> 315 us per layer of the 8B step.
# decode.hip measured slower with it (165.1 -> 167.3 us at 256 requests).
EXTRA_FLAGS = {
    "prefill.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
    "mixed.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
           "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in (p.stderr or "").splitlines() if noise not in ln)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stderr}")
    os.replace(tmp, out)


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES) + 1) as ex:
        objs = list(ex.map(_compile, SOURCES + [CEILING_SOURCE]))
    _link(objs[:-1], LIB)
    _link(objs[-1:], CEILING_LIB)
    if verbose:
        print(f"built {LIB} and {CEILING_LIB}")
    return LIB


if __name__ == "__main__":
    build()
