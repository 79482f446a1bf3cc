"""Address and undefined-behaviour sanitizers on the CPU side.

Two sanitizer builds, made here and run in child processes (the sanitizer
runtime must be the first library loaded, so it is preloaded there):
  * the C oracle (gcc -fsanitize=address,undefined), with every oracle pin
    of tests/test_oracle_pins.py run against it;
  * the library's host code (hipcc, -fsanitize=address,undefined applied to
    the host compilation only; the GPU code is built as usual), with every
    host-side argument check of tests/test_abi_cpu.py run against it.  Those
    calls are all rejected before any HIP call, so no GPU is needed.
Any sanitizer report aborts the child process and fails the test.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CSRC = os.path.join(ROOT, "commit_gated_delta_amd", "csrc")
SOURCES = ["gdn_window", "gdn_window_mfma", "gdn_kda", "gdn_kda_mfma",
           "gdn_prefill", "gdn_state"]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _child(code, env_extra, timeout=600):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(env_extra)
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=timeout)


def _undefined_symbols(lib):
    r = subprocess.run(["nm", "-D", "--undefined-only", lib],
                       capture_output=True, text=True, check=True)
    return r.stdout


@pytest.fixture(scope="module")
def oracle_san(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    out = str(tmp_path_factory.mktemp("san") / "liboracle_san.so")
    subprocess.run(
        ["gcc", "-O1", "-g", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
         "-fopenmp", "-fPIC", "-shared", "-std=c11", "-fno-fast-math",
         "-ffp-contract=off", "-o", out,
         os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-lm"], check=True)
    rt = subprocess.run(["gcc", "-print-file-name=libasan.so"],
                        capture_output=True, text=True).stdout.strip()
    return out, rt


@pytest.fixture(scope="module")
def library_san(tmp_path_factory):
    rts = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/"
                    "libclang_rt.asan-x86_64.so")
    if not os.path.exists(HIPCC) or not rts:
        pytest.skip("hipcc or its ASan runtime not available")
    d = tmp_path_factory.mktemp("san_lib")
    host_san = ["-Xarch_host", "-fsanitize=address",
                "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-omit-frame-pointer"]
    procs, objs = [], []
    for f in SOURCES:
        obj = str(d / (f + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen(
            [HIPCC, "-O1", "-g", "--offload-arch=gfx950", "-std=c++17",
             "-fPIC", "-ffp-contract=off", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", *host_san,
             "-Wno-unused-command-line-argument",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c",
             os.path.join(CSRC, f + ".hip"), "-o", obj],
            stdout=subprocess.DEVNULL, stderr=subprocess.PIPE, text=True))
    for p in procs:
        _, err = p.communicate(timeout=900)
        assert p.returncode == 0, err[-2000:]
    out = str(d / "libgdn_san.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
                    "-shared-libasan", *host_san[:4], "-o", out, *objs],
                   check=True)
    return out, rts[0]


def test_sanitizer_builds_are_instrumented(oracle_san, library_san):
    for lib in (oracle_san[0], library_san[0]):
        syms = _undefined_symbols(lib)
        assert "__asan_" in syms, lib
        assert "__ubsan_handle_" in syms, lib


def test_oracle_pins_under_address_and_ub_sanitizers(oracle_san):
    lib, rt = oracle_san
    code = ("import sys, oracle, pytest\n"
            "oracle.use_library(%r)\n"
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', "
            "'tests/test_oracle_pins.py']))\n" % lib)
    r = _child(code, {"LD_PRELOAD": rt})
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout


def test_host_argument_checks_under_address_and_ub_sanitizers(library_san):
    lib, rt = library_san
    code = ("import sys, pytest\n"
            "import commit_gated_delta_amd as gdn\n"
            "assert gdn.LIB_PATH == %r\n"
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', "
            "'tests/test_abi_cpu.py', '-k', 'not missing_library']))\n" % lib)
    r = _child(code, {"LD_PRELOAD": rt, "GDN_LIBRARY": lib})
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout
