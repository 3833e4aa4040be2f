"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code, on the CPU.

* The oracle (oracle/*.c) is built with gcc -fsanitize=address,undefined and the
  three pin suites run against it.
* The C-ABI's host side (fsl_api.cpp: argument validation, workspace and state
  layouts) is built with hipcc, the sanitizers on its host pass only, linked with
  the library's other objects, and test_abi_cpu.py runs against it (validation
  only: nothing is launched).
Each run is a subprocess with the sanitizer runtime preloaded and the library
chosen through FSL_ORACLE_LIBRARY / FSL_LIBRARY; any report fails the test.
"""
import glob
import os
import subprocess
import sys

import pytest

import cell_routed_long_amd as fsl
from cell_routed_long_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_DIR = os.path.join(ROOT, "oracle")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:exitcode=86",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=87"}


def _run_pytest(tests, env_extra, preload, tmp_path):
    env = dict(os.environ, **SAN_ENV, **env_extra, LD_PRELOAD=preload)
    res = subprocess.run([sys.executable, "-m", "pytest", *tests, "-q", "-x", "-p", "no:cacheprovider",
                          "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0 and "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    lib = tmp_path / "liboracle_san.so"
    srcs = sorted(glob.glob(os.path.join(ORACLE_DIR, "*.c")))
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-o", str(lib),
                           *srcs, "-lm"])
    asan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    ubsan = subprocess.check_output(["gcc", "-print-file-name=libubsan.so"], text=True).strip()
    _run_pytest(["tests/test_oracle_pins.py", "tests/test_fsb_oracle_pins.py", "tests/test_oracle_backward_pins.py"],
                {"FSL_ORACLE_LIBRARY": str(lib)}, f"{asan}:{ubsan}", tmp_path)


def test_abi_host_validation_under_asan_ubsan(tmp_path):
    runtimes = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not runtimes:
        pytest.skip("no clang AddressSanitizer runtime in this ROCm installation")
    objs = [os.path.join(_build.BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in _build.SOURCES
            if s != "fsl_api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        fsl.build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    api_o = tmp_path / "fsl_api.o"
    flags = [f for f in _build.COMMON_FLAGS if f != "-O3"]
    subprocess.check_call([_build.HIPCC, *flags, "-O1", "-g", "-fno-omit-frame-pointer", *san, "-c",
                           os.path.join(_build.CSRC, "fsl_api.cpp"), "-o", str(api_o)],
                          stderr=subprocess.DEVNULL)
    lib = tmp_path / "libfsl_san.so"
    subprocess.check_call([_build.HIPCC, f"--offload-arch={_build.ARCH}", "-shared", "-fPIC", "-shared-libsan", *san,
                           "-o", str(lib), *objs, str(api_o)])
    _run_pytest(["tests/test_abi_cpu.py"], {"FSL_LIBRARY": str(lib)}, runtimes[-1], tmp_path)
