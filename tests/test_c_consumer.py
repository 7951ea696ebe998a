"""include/qil.h as a plain C99 header: a C program (tests/c_consumer.c)
compiled by gcc with -std=c99 -pedantic -Werror, linked against libqil.so,
calls entry points whose argument checks fail before any HIP call and checks
the documented return codes (no GPU needed)."""

import os
import shutil
import subprocess
import tempfile

import pytest

import paged_kv_attention_16_amd as qil

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_c99_consumer_links_and_runs():
    lib = qil.lib_path()
    if not os.path.exists(lib):
        import __graft_entry__
        __graft_entry__.build()
    libdir = os.path.dirname(lib)
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "c_consumer")
        # link by path (the library is named libqil.so in the package directory)
        cmd = ["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
               "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "c_consumer.c"),
               "-o", exe, "-L", libdir, "-lqil", f"-Wl,-rpath,{libdir}"]
        p = subprocess.run(cmd, capture_output=True, text=True)
        assert p.returncode == 0, p.stderr
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stdout + r.stderr
        assert r.stdout.count("ok   ") == 5, r.stdout
