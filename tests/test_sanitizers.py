"""Sanitizer builds on the CPU (no GPU): the fp64 oracle (oracle/oracle.c) and
the host-side C ABI layer of the library (api.cpp, quantile.cpp, with the
device side stubbed) built with AddressSanitizer and UndefinedBehaviorSanitizer
by gcc/g++ and run on drivers under tests/sanitize/ that call every entry
point; any sanitizer report fails the test."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-D_DEFAULT_SOURCE", "-Wall", "-Wno-unknown-pragmas", *SAN, "-o", exe,
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-lm"])
    r = _run([exe], env=ENV, timeout=300)
    assert "0 failures" in r.stdout and "runtime error" not in r.stderr


@pytest.mark.skipif(not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"), reason="HIP headers missing")
def test_c_abi_host_layer_under_sanitizers(tmp_path):
    exe = str(tmp_path / "api_san")
    csrc = os.path.join(ROOT, "attention_spark_ffn_amd", "csrc")
    _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{ROOT}/include", f"-I{csrc}",
          "-Wall", *SAN, "-o", exe, os.path.join(csrc, "api.cpp"), os.path.join(csrc, "quantile.cpp"),
          os.path.join(ROOT, "tests", "sanitize", "api_driver.cpp")])
    r = _run([exe], env=ENV, timeout=120)
    assert "0 failures" in r.stdout and "runtime error" not in r.stderr
