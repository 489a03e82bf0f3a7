"""The library's host code under UndefinedBehaviorSanitizer (no GPU needed).

The C-ABI's host side (shape checks, launch planners, workspace layout) does
the size arithmetic every kernel relies on.  This builds a copy of the
library whose host code is instrumented with -fsanitize=undefined (device
code unchanged; every sanitizer flag applies to the host pass only), then runs
the planner sweep (some 14 k shapes up to T = 10^6, E = 4096, G = 32, k = 32)
and the ABI tests against it in a fresh process, so that any signed overflow,
bad shift or out-of-range conversion on those paths aborts the run.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from combine_ep_get_dispatch_amd import build as B  # noqa: E402

RUNTIME = "libclang_rt.ubsan_standalone-x86_64.so"


def _runtime_dir():
    base = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib", "llvm", "lib", "clang")
    if not os.path.isdir(base):
        return None
    for ver in sorted(os.listdir(base), reverse=True):
        d = os.path.join(base, ver, "lib", "linux")
        if os.path.exists(os.path.join(d, RUNTIME)):
            return d
    return None


RUNNER = """
import sys
sys.path.insert(0, {root!r})
from combine_ep_get_dispatch_amd import binding as B
B.load({lib!r})
import pytest
sys.exit(pytest.main(["-x", "-q", "-p", "no:cacheprovider",
                      {planner!r}, {abi!r}]))
"""


def test_host_code_under_ubsan(tmp_path):
    rt = _runtime_dir()
    if not os.path.exists(B.hipcc()) or rt is None:
        pytest.skip("hipcc or the UBSan runtime is not installed")
    lib = str(tmp_path / "libmoedisp_ubsan.so")
    host = ["-fsanitize=undefined", "-fno-sanitize-recover=all", "-shared-libsan", "-O1"]
    flags = [f for h in host for f in ("-Xarch_host", h)]
    B.build(out=lib, extra_flags=flags)
    code = RUNNER.format(root=ROOT, lib=lib, planner=os.path.join(ROOT, "tests", "test_planner_limits.py"),
                         abi=os.path.join(ROOT, "tests", "test_abi.py"))
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = rt + os.pathsep + env.get("LD_LIBRARY_PATH", "")
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "runtime error" not in r.stderr, r.stderr[-3000:]
