"""The C ABI's host code (argument checks, workspace plans, tiling) under
AddressSanitizer and UndefinedBehaviorSanitizer: a copy of the library with
its host pass instrumented (the device code is built as usual) is linked
into tests/host_abi_checks.c, which calls every entry point with valid and
invalid problems and fake device pointers that are never dereferenced (each
call returns before its first HIP call), so no GPU is needed."""
import os
import shlex
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "chunked_kl_loss_02_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
# host-pass sanitizers only: each -fsanitize= right after -Xarch_host
HOST_SAN = shlex.split("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                       "-Xarch_host -fno-sanitize-recover=undefined")

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                                reason="needs hipcc and ROCm's clang")


def test_host_abi_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    lib = tmp_path / "libkdkl_san.so"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-result",
                    *HOST_SAN, os.path.join(CSRC, "kd_host.hip"), "-o", str(lib)],
                   check=True, capture_output=True, text=True, timeout=600)
    exe = tmp_path / "host_abi_checks"
    subprocess.run([CLANG, "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "host_abi_checks.c"),
                    str(lib), f"-Wl,-rpath,{tmp_path}", "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
                    "-lm", "-o", str(exe)],
                   check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "host ABI checks: ok" in r.stdout
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
