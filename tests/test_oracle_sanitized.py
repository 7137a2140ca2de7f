"""The oracle under the host sanitizers: oracle/qoq_oracle.c is compiled with
AddressSanitizer and UndefinedBehaviorSanitizer (out-of-bounds accesses,
use-after-free, signed overflow, shifts past the width, misaligned loads all
abort the process), and the golden and property suites run against that
build in a subprocess. Host code only: nothing here touches a GPU."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_suites_pass_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    lib = tmp_path / "libqoq_oracle_san.so"
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           os.path.join(ROOT, "oracle", "qoq_oracle.c"), "-o", str(lib), "-lm"]
    subprocess.check_call(cmd)
    env = dict(os.environ)
    env.update({
        "QOQ_ORACLE_LIB": str(lib),
        "LD_PRELOAD": asan,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "OMP_NUM_THREADS": "4",
    })
    suites = [os.path.join(ROOT, "tests", f) for f in ("test_oracle_golden.py", "test_oracle_properties.py")]
    proc = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                           "-p", "no:cacheprovider", *suites],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=1500)
    tail = (proc.stdout + proc.stderr)[-4000:]
    assert proc.returncode == 0, tail
    assert "passed" in proc.stdout, tail
    # the suites ran on the sanitized build, with the sanitizer runtime active
    probe = ("import oracle, ctypes; lib = oracle._load(); "
             "assert lib._name == %r, lib._name; "
             "assert hasattr(ctypes.CDLL(None), '__asan_init'); print('sanitized')" % str(lib))
    chk = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=300)
    assert chk.returncode == 0 and "sanitized" in chk.stdout, chk.stdout + chk.stderr
