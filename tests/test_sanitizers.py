"""The host code under AddressSanitizer + UBSan and ThreadSanitizer (g++/gcc, CPU only).

* The C ABI layer (ggml_q2_dequant_amd/csrc/q2k_api.cpp with q2k_sizes.cpp),
  linked against tests/asan_stubs.cpp: host memory stands in for device
  memory and each launch stub touches exactly the bytes its kernel reads and
  writes. tests/api_asan_driver.cpp drives every entry point's accepted path
  with exactly-sized buffers, so a workspace or caller scratch sized below what
  its kernels use, or a kernel handed a range past a buffer, is a reported
  heap-buffer-overflow; the same driver under ThreadSanitizer runs calls from
  several host threads on shared and separate streams.
* The ABI rejection tests (tests/test_abi.py) and the GGUF reader tests, run
  in a child Python against the same layer built as a sanitized shared library.
* The oracle (oracle/q2k_oracle.c) built with the sanitizers and put through
  its pins (tests/test_oracle_pins.py, test_moe_oracle.py, test_sample_oracle.py)
  in a child Python.

Sanitizer reports go to files in a temporary directory; a test fails on a
nonzero exit or on any report. Never needed on a GPU machine.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
CSRC = os.path.join(ROOT, "ggml_q2_dequant_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")

SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer"]
ASAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
TSAN = ["-fsanitize=thread"]
CXX_FLAGS = ["-std=c++17", "-D__HIP_PLATFORM_AMD__", "-isystem", "/opt/rocm/include", "-I" + INCLUDE, "-I" + CSRC]
API_SOURCES = [os.path.join(CSRC, "q2k_api.cpp"), os.path.join(CSRC, "q2k_sizes.cpp"),
               os.path.join(TESTS, "asan_stubs.cpp")]


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def built(tmp_path_factory):
    if not shutil.which("g++") or not shutil.which("gcc"):
        pytest.skip("g++/gcc not available")
    if not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("HIP headers not available")
    d = tmp_path_factory.mktemp("san")
    out = {
        "api_asan": str(d / "api_asan"),
        "api_tsan": str(d / "api_tsan"),
        "lib_asan": str(d / "libq2k_asan.so"),
        "oracle_asan": str(d / "liboracle_asan.so"),
    }
    driver = os.path.join(TESTS, "api_asan_driver.cpp")
    jobs = [
        ["g++", *CXX_FLAGS, *SAN_FLAGS, *ASAN, *API_SOURCES, driver, "-pthread", "-o", out["api_asan"]],
        ["g++", *CXX_FLAGS, *SAN_FLAGS, *TSAN, *API_SOURCES, driver, "-pthread", "-o", out["api_tsan"]],
        ["g++", *CXX_FLAGS, *SAN_FLAGS, *ASAN, "-shared", "-fPIC", *API_SOURCES, os.path.join(CSRC, "q2k_gguf.cpp"),
         "-pthread", "-o", out["lib_asan"]],
        # The oracle's own flags (oracle.build) plus the sanitizers.
        ["gcc", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", *SAN_FLAGS, *ASAN,
         "-o", out["oracle_asan"], os.path.join(ROOT, "oracle", "q2k_oracle.c"), "-lm"],
    ]
    procs = [subprocess.Popen(j, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True) for j in jobs]
    for j, p in zip(jobs, procs):
        log, _ = p.communicate()
        assert p.returncode == 0, "%s\n%s" % (" ".join(j), log[-3000:])
    out["dir"] = str(d)
    return out


def _reports(d):
    found = []
    for f in sorted(glob.glob(os.path.join(d, "*san*"))):
        with open(f, errors="replace") as fh:
            found.append(f + ":\n" + fh.read()[-3000:])
    return found


def _run(cmd, report_dir, extra_env=None, preload=False):
    os.makedirs(report_dir, exist_ok=True)
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=%d:log_path=%s" % (0 if preload else 1, os.path.join(report_dir, "asan"))
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:log_path=%s" % os.path.join(report_dir, "ubsan")
    env["TSAN_OPTIONS"] = "halt_on_error=1:log_path=%s" % os.path.join(report_dir, "tsan")
    if preload:
        libs = [_runtime("libasan.so"), _runtime("libubsan.so")]
        if None in libs:
            pytest.skip("sanitizer runtimes not found")
        env["LD_PRELOAD"] = ":".join(libs)
    env.update(extra_env or {})
    res = subprocess.run(cmd, capture_output=True, text=True, env=env, cwd=TESTS, timeout=600)
    reports = _reports(report_dir)
    assert res.returncode == 0 and not reports, "rc=%d\n%s\n%s\n%s" % (
        res.returncode, res.stdout[-2000:], res.stderr[-2000:], "\n".join(reports))
    return res


def test_abi_layer_under_address_and_ub_sanitizers(built):
    res = _run([built["api_asan"]], os.path.join(built["dir"], "rep_api_asan"))
    assert res.stdout.startswith("ok ")
    checks, launches = map(int, res.stdout.split()[1:3])
    assert checks >= 200 and launches >= 250


def test_abi_layer_under_thread_sanitizer(built):
    res = _run([built["api_tsan"]], os.path.join(built["dir"], "rep_api_tsan"))
    assert res.stdout.startswith("ok ")


def test_abi_and_gguf_tests_against_the_sanitized_library(built):
    res = _run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                "test_abi.py", "test_gguf.py"],
               os.path.join(built["dir"], "rep_abi"), {"Q2K_ABI_TEST_LIB": built["lib_asan"]}, preload=True)
    assert " passed" in res.stdout and "failed" not in res.stdout


def test_oracle_pins_under_address_and_ub_sanitizers(built):
    env = {"Q2K_ORACLE_LIB": built["oracle_asan"]}
    probe = _run([sys.executable, "-c", "import sys; sys.path.insert(0, %r); import oracle; print(oracle._load()._name)"
                  % ROOT], os.path.join(built["dir"], "rep_oracle_probe"), env, preload=True)
    assert probe.stdout.strip() == built["oracle_asan"]
    res = _run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                "test_oracle_pins.py", "test_moe_oracle.py", "test_sample_oracle.py"],
               os.path.join(built["dir"], "rep_oracle"), env, preload=True)
    assert " passed" in res.stdout and "failed" not in res.stdout
