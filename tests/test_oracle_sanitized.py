"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
code only, no GPU): its pins run against a sanitized build, and a planted
out-of-bounds write is caught, which shows that the sanitized runs can see
one.  A compute-sanitizer run of the page's own code found an out-of-bounds
shared-memory read in its combine receiver ("MSCCLPP EP implementation -
#852", the commit notes of the intranode port); these runs are the CPU side
of that discipline."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(env, args, timeout=900):
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


def test_oracle_pins_pass_under_asan_and_ubsan(tmp_path):
    lib = oracle.compile_oracle(oracle.SRC, str(tmp_path / "liboracle_san.so"), sanitize=True)
    env = oracle.sanitizer_env(lib)
    r = _run(env, ["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_oracle_pins.py"])
    tail = (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail


def test_sanitized_oracle_catches_a_planted_overflow(tmp_path):
    """A one-past-the-end write in the layout's counter reset, planted in a
    copy of oracle.cpp: the sanitized build must abort with a heap overflow
    report when the layout runs on arrays numpy allocated."""
    src = open(oracle.SRC).read()
    old = "for (int e = 0; e < E; ++e) tokens_per_expert[e] = 0;"
    assert src.count(old) == 1
    bad = tmp_path / "oracle_overflow.cpp"
    bad.write_text(src.replace(old, "for (int e = 0; e <= E; ++e) tokens_per_expert[e] = 0;"))
    lib = oracle.compile_oracle(str(bad), str(tmp_path / "liboracle_bad.so"), sanitize=True)
    env = oracle.sanitizer_env(lib)
    prog = ("import numpy as np, oracle; "
            "idx = np.array([[0, 1], [2, 3]], np.int32); "
            "oracle.get().layout(idx, 4, 2); print('no report')")
    r = _run(env, ["-c", prog], timeout=120)
    assert r.returncode != 0, r.stdout + r.stderr
    assert "heap-buffer-overflow" in r.stderr, r.stderr[-3000:]
