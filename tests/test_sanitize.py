"""Host sanitizer tier (CPU): AddressSanitizer and UndefinedBehaviorSanitizer
builds of the C oracle (gcc) and of the library's host code (hipcc, the
sanitizers on the host side only; device code is compiled unoptimised, since
it never runs here), each driven by the CPU tests of that code in a child
process with the sanitizer runtime preloaded: the oracle's pin tests, and the
C-ABI boundary tests (every host-side argument check, the workspace-size
arithmetic, the status strings).  Any report aborts the child.  A planted
heap overflow first shows that each toolchain's sanitizer reports in this
environment."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHILD = os.path.join(ROOT, "tests", "sanitize_child.py")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}

OVERFLOW_C = r"""
#include <stdlib.h>
int main(int argc, char **argv) {
    (void)argv;
    int *a = (int *)malloc(4 * sizeof(int));
    a[argc + 3] = 1;          /* one past the end */
    int r = a[0];
    free(a);
    return r;
}
"""


def gcc_runtime() -> str:
    libs = [subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True,
                           text=True).stdout.strip() for n in ("libasan.so", "libubsan.so")]
    if not all(os.path.isabs(p) and os.path.exists(p) for p in libs):
        pytest.skip("gcc sanitizer runtimes not found")
    return ":".join(libs)


def clang_runtime() -> str:
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found or not os.path.exists(HIPCC):
        pytest.skip("ROCm clang sanitizer runtime not found")
    return found[-1]


def run_child(args, preload):
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV)
    return subprocess.run([sys.executable, *args], capture_output=True, text=True, env=env,
                          timeout=600)


def test_gcc_sanitizer_reports_a_planted_overflow(tmp_path):
    src = tmp_path / "overflow.c"
    src.write_text(OVERFLOW_C)
    exe = tmp_path / "overflow"
    subprocess.run(["gcc", "-g", "-fsanitize=address,undefined", "-o", str(exe), str(src)],
                   check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True,
                         env=dict(os.environ, **SAN_ENV))
    assert res.returncode != 0 and "heap-buffer-overflow" in res.stderr


def test_clang_host_sanitizer_reports_a_planted_overflow(tmp_path):
    clang_runtime()
    src = tmp_path / "overflow.hip"
    src.write_text(OVERFLOW_C)
    exe = tmp_path / "overflow"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-g", "-o", str(exe), str(src)], check=True,
                   capture_output=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True,
                         env=dict(os.environ, **SAN_ENV))
    assert res.returncode != 0 and "heap-buffer-overflow" in res.stderr


def test_oracle_pins_under_asan_ubsan(tmp_path):
    preload = gcc_runtime()
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-o", str(lib),
                    os.path.join(ROOT, "oracle", "oracle.c"), "-lm"], check=True)
    res = run_child([CHILD, "oracle", str(lib)], preload)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out


def test_boundary_under_asan_ubsan(tmp_path):
    preload = clang_runtime()
    lib = tmp_path / "libpagedkv_san.so"
    cmd = [HIPCC, "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
           "-Xarch_host", "-O1", "-Xarch_device", "-O0", "-Xarch_host", "-g",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "paged_kv_cache_100_amd", "csrc"),
           "-o", str(lib), os.path.join(ROOT, "paged_kv_cache_100_amd", "csrc", "pagedkv.hip")]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    res = run_child([CHILD, "boundary", str(lib)], preload)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out
