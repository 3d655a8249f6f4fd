"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

sv_api.cpp (argument checks, launch planning, workspace arithmetic, the
allocation-free entry point's size checks) is compiled with host-only
sanitizers (`-Xarch_host -fsanitize=...`; the device code is untouched) and
linked with stand-in launchers (tests/sanitizer_stubs.cpp) into a library of
its own; test_abi_host.py then runs against that library in a child process
that preloads the sanitizer runtime.  Any out-of-bounds access, overflow or
other undefined behaviour on those paths aborts the child.  Runs on the CPU.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_abi_host_checks_under_sanitizers(tmp_path):
    rt = _asan_runtime()
    if not os.path.exists(HIPCC) or rt is None:
        pytest.skip("hipcc or the sanitizer runtime not found")
    api = os.path.join(ROOT, "draft_token_verification_sv_amd", "csrc", "sv_api.cpp")
    stubs = os.path.join(ROOT, "tests", "sanitizer_stubs.cpp")
    common = ["-O1", "-g", "-std=c++17", "-fPIC", *SAN]
    subprocess.run([HIPCC, "--offload-arch=gfx950", *common, "-x", "hip", "-c", api, "-o", str(tmp_path / "api.o")],
                   check=True, capture_output=True)
    subprocess.run([HIPCC, *common, "-c", stubs, "-o", str(tmp_path / "stubs.o")], check=True, capture_output=True)
    lib = tmp_path / "libsv_sanitized.so"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan", *SAN,
                    str(tmp_path / "api.o"), str(tmp_path / "stubs.o"), "-o", str(lib)], check=True, capture_output=True)
    syms = subprocess.run(["nm", "-D", str(lib)], check=True, capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "library not instrumented"
    env = dict(os.environ, SV_ABI_LIB=str(lib), LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_host.py"), "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"], env=env, capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    print(r.stdout[-3000:], r.stderr[-3000:])
    assert r.returncode == 0
    assert "passed" in r.stdout and "failed" not in r.stdout
