"""Host sanitizers (address and undefined behaviour) on the CPU oracle and on
the C ABI's host code.  The oracle is built with gcc and the sanitizers and
driven through every entry point on small seeded inputs (leak checks on).
The C ABI (api.cpp) is built for the host with the sanitizers, linked with
test stand-ins for the kernel launchers (tests/sanitize/launch_stubs.cpp),
and driven through its validation paths, a launch that fails and the check
mode.  No GPU is used; the GPU code itself is covered by the parity tests."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = os.path.join(HERE, "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, env=None, cwd=None):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, cwd=cwd, timeout=600)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    _run(["gcc", "-std=c99", "-O1", "-g", "-ffp-contract=off", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", os.path.join(SAN, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "sharq_oracle.c"), "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = _run([exe], env=env)
    assert r.stdout.strip().endswith("ok")


@pytest.mark.skipif(not all(os.path.exists(p) for p in (HIPCC, CLANG, CLANGXX)), reason="ROCm compilers not available")
def test_abi_host_code_under_address_and_undefined_sanitizers(tmp_path):
    flags = ["-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined"]
    api_o, stub_o, drv_o = (str(tmp_path / n) for n in ("api.o", "stubs.o", "drv.o"))
    _run([HIPCC] + flags + ["-c", os.path.join(ROOT, "sparsity_prep_amd", "csrc", "api.cpp"), "-o", api_o])
    _run([HIPCC] + flags + ["-c", os.path.join(SAN, "launch_stubs.cpp"), "-o", stub_o])
    _run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-c",
          os.path.join(SAN, "api_driver.c"), "-o", drv_o])
    exe = str(tmp_path / "api_asan")
    _run([CLANGXX, "-fsanitize=address,undefined", drv_o, api_o, stub_o, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("SHARQ_DEBUG", None)
    r = _run([exe], env=env)
    assert r.stdout.strip().endswith("ok")
    assert "sharq: sharq_linear:" in r.stderr  # the check mode names the failing entry point
