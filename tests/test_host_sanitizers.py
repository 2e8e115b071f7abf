"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

1. The oracle (oracle/oracle.c) built with gcc -fsanitize=address,undefined and
   driven through every entry point by tests/sanitize/oracle_check.c.
2. The library's host code (csrc/llama_abi.cpp: validation, sizing, handles,
   refusals) built with the sanitizers on the host side only, linked with the
   kernels' objects as built, and walked by tests/sanitize/abi_host_check.c
   through sizing, loading, cache handles and the refusal of bad arguments --
   paths that enqueue nothing, so no GPU is needed.

Either sanitizer aborts the program on the first invalid access, leak or
undefined operation, so a zero exit status is the check."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "_build", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

ENV = dict(os.environ,
           ASAN_OPTIONS="abort_on_error=0:halt_on_error=1:detect_leaks=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-3000:] + r.stderr[-6000:]
    return r


def test_oracle_under_sanitizers():
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_check")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall",
          "-Wno-unknown-pragmas", f"-I{os.path.join(ROOT, 'oracle')}",
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "oracle_check.c"),
          "-o", exe, "-lm"])
    r = _run([exe], env=ENV, timeout=300)
    assert "oracle check ok" in r.stdout


def test_library_host_code_under_sanitizers():
    if shutil.which("hipcc") is None:
        pytest.skip("no hipcc")
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_llama_lib_build", os.path.join(ROOT, "dense_gqa_llama_amd", "build.py"))
    lb = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(lb)
    kernels = [s for s in lb.sources() if s.endswith(".hip")]
    objs = [os.path.join(lb.OBJ, os.path.basename(s) + ".o") for s in kernels]
    if not all(os.path.exists(o) for o in objs):
        lb.build()
    os.makedirs(OUT, exist_ok=True)
    abi = os.path.join(lb.CSRC, "llama_abi.cpp")
    abi_obj = os.path.join(OUT, "llama_abi_asan.o")
    drv_obj = os.path.join(OUT, "abi_host_check.o")
    exe = os.path.join(OUT, "abi_host_check")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    _run(["hipcc", *[f for f in lb.FLAGS if f != "-O3"], "-O1", "-g", *san, "-x", "hip", "-c", abi,
          "-o", abi_obj])
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    _run([clang, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          f"-I{os.path.join(ROOT, 'include')}", "-c", os.path.join(HERE, "abi_host_check.c"),
          "-o", drv_obj])
    _run([clang + "++", "-fsanitize=address,undefined", drv_obj, abi_obj, *objs,
          f"-L{os.path.join(ROCM, 'lib')}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}",
          "-lamdhip64", "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert "abi host check ok" in r.stdout
