"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

`oracle/sanitize_driver.c` links `oracle/mpfa_oracle.c` into a standalone
program (no Python, no preloaded runtime) and calls every exported oracle
function on small and edge-case inputs; built with gcc's address and
undefined-behaviour sanitizers (float-to-int overflow included, every report
fatal), it must run to completion with no report and all of its own checks
passing."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")
SANITIZE = "-fsanitize=address,undefined,float-cast-overflow"


def _build(tmp_path, extra):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_sanitized")
    cmd = [gcc, "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", *extra,
           "-o", exe, os.path.join(ORACLE, "mpfa_oracle.c"),
           os.path.join(ORACLE, "sanitize_driver.c"), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr + r.stdout).lower():
        pytest.skip(f"sanitizer runtime not available: {r.stderr.strip()[:200]}")
    assert r.returncode == 0, r.stderr
    return exe


def _run(exe, leaks):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = f"detect_leaks={1 if leaks else 0}:abort_on_error=0:exitcode=23"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=24"
    env["OMP_NUM_THREADS"] = "4"
    return subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)


@pytest.mark.parametrize("openmp", [False, True], ids=["serial", "openmp"])
def test_oracle_runs_clean_under_asan_and_ubsan(tmp_path, openmp):
    extra = [SANITIZE, "-fno-sanitize-recover=all"] + (["-fopenmp"] if openmp else [])
    exe = _build(tmp_path, extra)
    # leak checking needs ptrace, which some containers forbid: fall back to
    # ASan without it only when LeakSanitizer itself says it cannot run
    r = _run(exe, leaks=True)
    if r.returncode != 0 and "LeakSanitizer has encountered a fatal error" in r.stderr:
        r = _run(exe, leaks=False)
    assert r.returncode == 0, f"exit {r.returncode}\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "runtime error" not in r.stderr, r.stderr[-4000:]
    assert "all checks passed" in r.stdout
