"""The oracle's pin suite (tests/test_oracle.py) against a build of
oracle/oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer (gcc,
host code only), in a subprocess that preloads the sanitizer runtimes.  A
control plants an out-of-bounds read (one element past a row) in a copy of
the oracle and checks that the sanitized run reports it, so a clean run
means the sanitizers were live."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _build(src, out):
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                           "-fno-fast-math", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", "-o", out, src, "-lm"])
    return out


def _run_pins(lib):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    env = dict(os.environ, ORACLE_LIB=lib, LD_PRELOAD=f"{asan} {ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_oracle.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


@pytest.fixture(scope="module", autouse=True)
def _need_runtimes():
    if not (_runtime("libasan.so") and _runtime("libubsan.so")):
        pytest.skip("gcc sanitizer runtimes not installed")


def test_pins_pass_under_asan_and_ubsan(tmp_path):
    r = _run_pins(_build(SRC, str(tmp_path / "liboracle_san.so")))
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]


def test_sanitizer_catches_a_planted_overread(tmp_path):
    src = open(SRC).read()
    old = "for (int64_t v = 0; v < V; ++v) R += r[v];"
    assert src.count(old) == 1
    bad = tmp_path / "oracle_overread.c"
    bad.write_text(src.replace(old, "for (int64_t v = 0; v <= V; ++v) R += r[v];"))
    r = _run_pins(_build(str(bad), str(tmp_path / "liboracle_overread.so")))
    assert r.returncode != 0 and "heap-buffer-overflow" in (r.stdout + r.stderr)
