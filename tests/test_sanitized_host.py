"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds, each exercised by an existing CPU test file in a subprocess:
  * the oracle (oracle/paro_ref.c) with gcc, without OpenMP (the plain C
    build must work too) and with -fsanitize=address,undefined, under the
    oracle's pin suite;
  * libparo's host-side ABI layer (argument validation, workspace layout,
    path choice: csrc/paro_abi.cpp) compiled with the sanitizers on its host
    pass only, linked with the kernel objects of the regular build, under
    the C-ABI checks that need no GPU.
Any sanitizer report aborts the subprocess, which fails the test.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

from oracle import ref

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _gcc_runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _run_pytest(test_file, env):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", test_file],
                       env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, f"exit {r.returncode}:\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"


def test_oracle_without_openmp_under_sanitizers(tmp_path):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = str(tmp_path / "libparo_ref_san.so")
    ref.build(lib, openmp=False, extra=["-O1", "-g", *SAN])
    env = dict(os.environ, PARO_REF_LIB=lib, LD_PRELOAD=f"{asan}:{ubsan}", ASAN_OPTIONS="detect_leaks=0")
    _run_pytest(os.path.join(HERE, "test_oracle_pins.py"), env)


def test_abi_layer_under_sanitizers(tmp_path):
    from rotation_int4_weight_amd import build as libbuild
    kernels = [src for src in libbuild.SOURCES if src != "paro_abi.cpp"]
    objs = [os.path.join(libbuild.BUILD, k + ".o") for k in kernels]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("kernel objects of the regular build are missing (run the build first)")
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    clangxx = "/opt/rocm/llvm/bin/clang++"
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not rt or not os.path.exists(clangxx) or not os.path.exists(hipcc):
        pytest.skip("ROCm clang sanitizer runtime not found")
    obj = str(tmp_path / "paro_abi.o")
    host_san = []
    for f in SAN:  # sanitizers on the host pass only
        host_san += ["-Xarch_host", f]
    subprocess.run([hipcc, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", *host_san,
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "rotation_int4_weight_amd", "csrc"),
                    "-c", os.path.join(ROOT, "rotation_int4_weight_amd", "csrc", "paro_abi.cpp"), "-o", obj],
                   check=True, capture_output=True)
    lib = str(tmp_path / "libparo_san.so")
    rtdir = os.path.dirname(rt[-1])
    subprocess.run([clangxx, "-shared", "-fPIC", obj, *objs, "-L", rtdir, "-lclang_rt.asan-x86_64",
                    "-Wl,-rpath," + rtdir, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", lib],
                   check=True, capture_output=True)
    env = dict(os.environ, PARO_LIB=lib, LD_PRELOAD=rt[-1], ASAN_OPTIONS="detect_leaks=0")
    _run_pytest(os.path.join(HERE, "test_abi_cpu.py"), env)
