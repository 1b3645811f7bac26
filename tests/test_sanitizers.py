"""Host-side memory and undefined-behaviour checks (AddressSanitizer and
UndefinedBehaviorSanitizer, CPU only).

Two sanitized builds are made in a temporary folder with gcc/g++:
  * the fp64 oracle (oracle/kda_oracle.c), under which the oracle's own pin
    tests (test_oracle.py, test_oracle_bwd.py) run;
  * the library's C-ABI validation layer (csrc/kda_api.cpp), linked with the
    regular objects of the HIP kernels, under which the ABI tests
    (test_abi.py: every export, every argument-validation path, the status
    word mapping) run. No GPU is touched.
Each run is a child pytest process with the sanitizer runtime preloaded
(Python itself is not instrumented); any sanitizer report fails the test.
"""
import glob
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.sanitize

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_46_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]


def _libasan():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return path


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])


def _child_pytest(files, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = _libasan()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["OMP_NUM_THREADS"] = env.get("OMP_NUM_THREADS", "4")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *files]
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    out = r.stdout + r.stderr
    print(out[-2000:])
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]


@pytest.fixture(scope="module")
def sandir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("sanitized"))


def test_oracle_under_sanitizers(sandir):
    lib = os.path.join(sandir, "libkda_oracle_san.so")
    _run(["gcc", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra", *SAN, "-o", lib,
          os.path.join(ROOT, "oracle", "kda_oracle.c")])
    _child_pytest(["tests/test_oracle.py", "tests/test_oracle_bwd.py"], {"KDA_ORACLE_LIB": lib})


def test_abi_validation_under_sanitizers(sandir):
    # every kernel object the regular build makes (all of build.py's sources but the API layer)
    from gated_delta_rule_46_amd import build as b
    objs = [os.path.join(ROOT, "gated_delta_rule_46_amd", "_build", os.path.splitext(f)[0] + ".o")
            for f in b.SOURCES if f != "kda_api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        from gated_delta_rule_46_amd import build
        build.build()
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    api = os.path.join(sandir, "kda_api_san.o")
    _run(["g++", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(rocm, "include"),
          "-I" + os.path.join(ROOT, "include"), "-Wall", *SAN, "-c", os.path.join(CSRC, "kda_api.cpp"), "-o", api])
    lib = os.path.join(sandir, "libkda_san.so")
    _run(["g++", "-shared", "-fPIC", "-fsanitize=address,undefined", "-o", lib, api, *objs,
          "-L" + os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib")])
    _child_pytest(["tests/test_abi.py"], {"KDA_LIB": lib})
