"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): the library is rebuilt with both sanitizers on its host code
(tests/host_sanitizer.py), and every test of tests/test_abi.py -- the
exports, each entry point's argument checks with every error code, the split
plans and workspace sizes -- runs against it in a child process with the
ASan runtime preloaded.  Any out-of-bounds access, use after free or
undefined behaviour in that code aborts the child with the sanitizer's
report."""

import glob
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

from host_sanitizer import asan_runtime, build_sanitized  # noqa: E402


def test_abi_under_host_sanitizers():
    lib = build_sanitized()
    logs = tempfile.mkdtemp(prefix="qil_sanitizer_")
    env = dict(os.environ)
    # the ASan runtime has to come first among the preloaded libraries
    env["LD_PRELOAD"] = ":".join(p for p in (asan_runtime(), env.get("LD_PRELOAD", "")) if p)
    # reports go to files under `logs` (a dying child's stderr can be lost)
    env["ASAN_OPTIONS"] = f"detect_leaks=0:halt_on_error=1:exitcode=97:log_path={logs}/asan"
    env["UBSAN_OPTIONS"] = f"halt_on_error=1:print_stacktrace=1:log_path={logs}/ubsan"
    env["QIL_ABI_LIB"] = lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi.py")],
                       env=env, capture_output=True, text=True, timeout=900, cwd=os.path.dirname(HERE))
    reports = "".join(open(f).read() for f in sorted(glob.glob(os.path.join(logs, "*"))))
    out = reports[-4000:] + r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, out
    assert reports == "", out
    assert " passed" in r.stdout, out
