"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no GPU).

The C oracle is rebuilt with both sanitizers and its pinned tests run against that build;
librtp.so's host side (argument checks, size queries, status strings, the exported-symbol
list) is rebuilt with both sanitizers on the host pass and the ABI tests run against it.
Each run is a child process that preloads the matching runtime (gcc's libasan for the
oracle, clang's for librtp) and names the instrumented library in the loader's override
variable.  A planted out-of-bounds write into the oracle shows that the instrumentation is
live: it must end the child with an AddressSanitizer report.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

ASAN_OPTIONS = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
UBSAN_OPTIONS = "print_stacktrace=1:halt_on_error=1"


def _gcc_asan():
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not installed")
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's libasan is not installed")
    return path


def _clang_asan():
    from head_wise_sparse_rtp_amd import build
    path = subprocess.run([build.HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                          capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("clang's ASan runtime is not installed")
    return path


def _child(args, env_extra, timeout=600):
    env = dict(os.environ, ASAN_OPTIONS=ASAN_OPTIONS, UBSAN_OPTIONS=UBSAN_OPTIONS, **env_extra)
    return subprocess.run([sys.executable] + args, cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=timeout)


@pytest.fixture(scope="module")
def oracle_san(tmp_path_factory):
    import oracle
    runtime = _gcc_asan()
    out = str(tmp_path_factory.mktemp("san") / "liboracle_san.so")
    oracle.build_sanitized(out)
    return {"RTP_ORACLE_LIBRARY": out, "LD_PRELOAD": runtime}


def test_oracle_tests_pass_under_sanitizers(oracle_san):
    probe = _child(["-c", "import oracle; print(oracle.lib()._name)"], oracle_san)
    assert probe.returncode == 0, probe.stderr[-3000:]
    assert probe.stdout.strip() == oracle_san["RTP_ORACLE_LIBRARY"]
    r = _child(["-m", "pytest", "tests/test_oracle.py", "-x", "-q", "-p", "no:cacheprovider"],
               oracle_san)
    assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-3000:])
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


def test_planted_overflow_is_reported(oracle_san):
    # 40 logits with equal cells select all 40 tokens; the index buffer holds 8
    code = (
        "import ctypes, numpy as np, oracle\n"
        "L = oracle.lib()\n"
        "z = np.zeros(40, dtype=np.float32)\n"
        "sel = np.zeros(8, dtype=np.int32)\n"
        "hist = np.zeros(256, dtype=np.float64)\n"
        "A = ctypes.c_int64(); b = ctypes.c_int32()\n"
        "L.rtpo_topp_select(z.ctypes.data, 40, 0.9, 1.0, sel.ctypes.data, hist.ctypes.data,\n"
        "                   ctypes.byref(A), ctypes.byref(b))\n"
        "print('no report')\n")
    r = _child(["-c", code], oracle_san)
    assert r.returncode != 0 and "no report" not in r.stdout
    assert "AddressSanitizer" in r.stderr and "heap-buffer-overflow" in r.stderr


def test_abi_tests_pass_with_sanitized_host_code(tmp_path):
    from head_wise_sparse_rtp_amd import build
    runtime = _clang_asan()
    out = str(tmp_path / "librtp_san.so")
    build.build_host_sanitized(out)
    env = {"RTP_LIBRARY": out, "LD_PRELOAD": runtime}
    probe = _child(["-c", "import head_wise_sparse_rtp_amd as m; print(m.lib()._name)"], env)
    assert probe.returncode == 0, probe.stderr[-3000:]
    assert probe.stdout.strip() == out
    r = _child(["-m", "pytest", "tests/test_abi.py", "-x", "-q", "-p", "no:cacheprovider"], env)
    assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-3000:])
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
