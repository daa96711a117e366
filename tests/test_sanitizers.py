"""CPU sanitizer runs: the oracle's pins with an AddressSanitizer + UndefinedBehaviorSanitizer
build of oracle.c (gcc), and the C ABI's host-side checks (test_abi.py) with a build of the
library whose host code (argument checks, workspace planning, status strings) is instrumented
the same way (hipcc, host pass only; the GPU code objects are the ordinary ones).  Each run is
a subprocess with the sanitizer runtime preloaded, stopping at the first report."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run_pytest(test_file, env_extra, tmp_path):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", test_file),
                        "-x", "-q", "-p", "no:cacheprovider"], cwd=str(tmp_path), env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout


def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    so = tmp_path / "liboracle_san.so"
    subprocess.check_call(["gcc", "-O1", "-g", "-fPIC", "-shared", "-fopenmp", "-std=c11",
                           "-fno-fast-math", "-ffp-contract=off", "-Wall",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fno-omit-frame-pointer", "-o", str(so),
                           os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    _run_pytest("test_oracle_pins.py", {"TCS_ORACLE_LIB": str(so), "LD_PRELOAD": asan}, tmp_path)


def test_abi_host_checks_under_asan_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from top_chunk_sparse_amd import build
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt or not os.path.exists(build.HIPCC):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined",
                "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
    host_files = ("api.cpp", "noalloc.hip")
    objs = []
    for src in build.SOURCES:
        if src in host_files:
            objs.append(build._compile(src, host_san, objdir=str(tmp_path)))
            continue
        obj = os.path.join(build.OBJDIR, src + ".o")
        if not (os.path.exists(obj) and
                os.path.getmtime(obj) >= os.path.getmtime(os.path.join(build.CSRC, src))):
            obj = build._compile(src, (), objdir=str(tmp_path))   # no current object: build one
        objs.append(obj)
    lib = str(tmp_path / "libtcsparse_san.so")
    subprocess.check_call([build.HIPCC, "--offload-arch=" + build.ARCH, "-shared", "-fPIC", "-o",
                           lib] + objs)
    _run_pytest("test_abi.py", {"TCS_LIB_PATH": lib, "LD_PRELOAD": rt[-1]}, tmp_path)
