"""The CPU oracle and the library's host layer (argument validation and
workspace plans in csrc/api.cpp) built with AddressSanitizer and
UndefinedBehaviorSanitizer, then driven by the existing CPU tests in a child
process: any out-of-bounds access, use after free, signed overflow or other
undefined behaviour on those paths aborts the child and fails the test.

Only host code is instrumented: the kernels' objects are linked in
unchanged and no GPU is used (the ABI tests stop at validation).
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _runtime(name):
    path = subprocess.check_output(["gcc", f"-print-file-name={name}"], text=True).strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"{name} not found")
    return path


def _child_env(**extra):
    env = dict(os.environ)
    env.update(extra)
    env["LD_PRELOAD"] = _runtime("libasan.so") + " " + _runtime("libubsan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    return env


def _pytest_child(env, files, tmp_path):
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
           "-m", "not gpu", *files]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    log = tmp_path / "child.log"
    log.write_text(r.stdout + "\n---- stderr ----\n" + r.stderr)
    assert r.returncode == 0, f"sanitized run failed (rc {r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr
    return r.stdout


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    lib = tmp_path / "liboracle_san.so"
    subprocess.check_call(["gcc", "-O1", "-g", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
                           "-fno-fast-math", *SAN, os.path.join(ROOT, "oracle", "hata_oracle.c"),
                           os.path.join(ROOT, "oracle", "hash_train_oracle.c"),
                           "-o", str(lib), "-lm"])
    out = _pytest_child(_child_env(HATA_ORACLE_LIB=str(lib)),
                        ["tests/test_oracle.py", "tests/test_oracle_bits.py",
                         "tests/test_oracle_recall.py", "tests/test_oracle_train.py"], tmp_path)
    assert " passed" in out


def test_host_validation_under_address_and_ub_sanitizers(tmp_path):
    from hash_top_sparse_encode_amd import _build
    objs = [os.path.join(_build.BUILD_DIR, s.rsplit(".", 1)[0] + ".o")
            for s in _build.SOURCES if s != "api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        _build.build()
    api_o = tmp_path / "api_san.o"
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-g", "-fPIC", *SAN, "-D__HIP_PLATFORM_AMD__",
                           "-I/opt/rocm/include",
                           "-c", os.path.join(_build.CSRC, "api.cpp"), "-o", str(api_o)])
    lib = tmp_path / "libhata_san.so"
    subprocess.check_call(["g++", "-shared", *SAN[:1], str(api_o), *objs, "-L/opt/rocm/lib",
                           "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(lib)])
    out = _pytest_child(_child_env(HATA_LIB_PATH=str(lib)), ["tests/test_abi.py"], tmp_path)
    assert " passed" in out
