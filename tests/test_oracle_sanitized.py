"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host code
only): szref.c is compiled with both, and every pin in oracle_pins runs
against that build in a child process with the ASan runtime preloaded.  An
out-of-bounds access, a use of freed memory, a shift past the width of its
operand, a signed overflow or a misaligned access ends the child with an
error; the pins must also still pass.  This keeps the values the oracle is
pinned to from resting on behaviour C leaves undefined."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "szref.c")

RUNNER = r"""
import sys
sys.path[:0] = [sys.argv[2], sys.argv[3]]
import numpy as np
import oracle, oracle_pins
O = oracle.OracleLib(sys.argv[1])
for check in oracle_pins.ALL_CHECKS:
    check(O)
    print("ok", check.__name__, flush=True)
# round trips over buffers sized exactly, so that any read or write past
# either end lands in an ASan redzone
rng = np.random.default_rng(7)
for n in (0, 1, 2, 3, 17, 4096, 65537):
    words = rng.integers(0, 65536, n, dtype=np.uint16)
    c = O.encode(words)
    exact = np.array(c, copy=True)
    out = np.empty(n, dtype=np.uint16)
    assert np.array_equal(O.decode(exact, n, out), words), n
    for cut in (1, 5):
        if exact.size > cut:
            st, _ = O.decode_status(np.array(exact[:-cut], copy=True), n)
            assert st != 0, (n, cut)
print("ALL PASSED", flush=True)
"""


def sanitizer_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.timeout(600)
def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan = sanitizer_runtime()
    if asan is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    lib = tmp_path / "libszref_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-Wall", "-Wextra", "-Werror", "-fPIC",
                    "-shared", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-o", str(lib), SRC], check=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=23"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=24"
    r = subprocess.run([sys.executable, "-c", RUNNER, str(lib), ROOT, os.path.join(ROOT, "tests")],
                       capture_output=True, text=True, env=env, timeout=540)
    tail = (r.stdout[-3000:] + "\n" + r.stderr[-3000:])
    assert r.returncode == 0, tail
    assert "ALL PASSED" in r.stdout, tail
    assert "runtime error" not in r.stderr, tail
