"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer, on
the CPU: the float64 oracle (oracle/attention_oracle.c) and the C ABI's host
side (argument validation, tile and split choice, size arithmetic of every
entry point in online_softmax_03_amd/csrc/*_api.hip, linked against empty
kernel tables so no call reaches a launch). Each is built into a driver
program (tests/sanitize/) and run; a sanitizer report fails the test. GPU
code is not instrumented: only the host pass of the HIP sources is."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "online_softmax_03_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
HOST_SOURCES = ["fa_api.hip", "bwd_api.hip", "fp8_api.hip", "softmax_api.hip", "noalloc_api.hip", "status.hip"]


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return r


def _check_clean(r, what):
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, f"{what}:\n{out[-4000:]}"
    assert r.returncode == 0, f"{what} exited {r.returncode}:\n{out[-4000:]}"


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "oracle_san")
        r = _run(["gcc", "-O1", "-std=c11", "-fopenmp", *SAN_FLAGS, "-o", exe,
                  os.path.join(SAN, "oracle_driver.c"), "-lm"])
        assert r.returncode == 0, r.stderr[-4000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
        _check_clean(_run([exe], env=env), "oracle driver")


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="needs the ROCm toolchain")
def test_capi_host_code_under_asan_ubsan():
    with tempfile.TemporaryDirectory() as tmp:
        objs = []
        procs = []
        srcs = [os.path.join(CSRC, f) for f in HOST_SOURCES] + [os.path.join(SAN, "tables_stub.hip")]
        for src in srcs:
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            # host pass instrumented only; the device pass of these files holds
            # no kernel (the fixed scratch array at most)
            cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-g",
                   "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                   "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", src, "-o", obj]
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
            objs.append(obj)
        for src, p in procs:
            _, err = p.communicate(timeout=600)
            assert p.returncode == 0, f"{src}:\n{err[-4000:]}"
        drv = os.path.join(tmp, "capi_driver.o")
        r = _run(["/opt/rocm/llvm/bin/clang", "-std=c11", "-O1", "-g", *SAN_FLAGS, "-I", os.path.join(ROOT, "include"),
                  "-c", os.path.join(SAN, "capi_driver.c"), "-o", drv])
        assert r.returncode == 0, r.stderr[-4000:]
        exe = os.path.join(tmp, "capi_san")
        r = _run([CLANGXX, *SAN_FLAGS, "-o", exe, drv, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                  "-Wl,-rpath,/opt/rocm/lib", "-lm"])
        assert r.returncode == 0, r.stderr[-4000:]
        # the HIP runtime is not instrumented and keeps allocations until exit
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
        _check_clean(_run([exe], env=env), "C ABI driver")
