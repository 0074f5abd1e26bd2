"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

abi.cpp (argument validation, workspace carve-up, scratch lookup, launches) is
compiled with the sanitizers on its host code only (hipcc -Xarch_host
-fsanitize=...; device code untouched) and linked with the library's other objects.
Then the plain-C ABI program (tests/abi_from_c.c, built with the same clang and
sanitizers) and the Python ABI tests (tests/test_abi.py, with the sanitizer runtime
preloaded and AB_ATTN_LIBRARY naming the sanitized build) must run clean: every
call there fails its host checks, so no GPU is needed."""

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_ibcs_amd", "csrc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
       "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    from block_sparse_attention_ibcs_amd import build as b

    rt = _asan_runtime()
    clang = "/opt/rocm/llvm/bin/clang"
    if rt is None or not os.path.exists(clang):
        pytest.skip("clang's sanitizer runtime is not available")
    out = tmp_path_factory.mktemp("asan")
    objs = []
    for src in b.SOURCES:
        obj = os.path.join(b.BUILD, os.path.splitext(src)[0] + ".o")
        if src != "abi.cpp":
            if not os.path.exists(obj):
                b.build()
            objs.append(obj)
    abi_o = str(out / "abi_san.o")
    subprocess.run([b.hipcc(), *b.FLAGS, "-O1", "-g", *SAN, "-x", "hip", "-c", os.path.join(CSRC, "abi.cpp"),
                    "-o", abi_o], check=True, capture_output=True, text=True)
    lib = str(out / "libabattn_san.so")
    # host link (the objects already carry their device code) with the host clang
    rocm_lib = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
    subprocess.run([clang + "++", "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libsan", abi_o, *objs,
                    "-L" + rocm_lib, "-lamdhip64", "-Wl,-rpath," + rocm_lib, "-o", lib],
                   check=True, capture_output=True, text=True)
    return {"lib": lib, "rt": rt, "clang": clang, "dir": str(out)}


def _env(rt):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


def test_c_program_under_sanitizers(sanitized):
    exe = os.path.join(sanitized["dir"], "abi_from_c_san")
    subprocess.run([sanitized["clang"], "-std=c99", "-g", "-fsanitize=address,undefined", "-shared-libsan",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_from_c.c"), sanitized["lib"],
                    "-Wl,-rpath," + os.path.dirname(sanitized["lib"]), "-Wl,-rpath," + os.path.dirname(sanitized["rt"]),
                    "-o", exe], check=True, capture_output=True, text=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=_env(sanitized["rt"]))
    assert res.returncode == 0, res.stderr[-3000:]
    assert "all checks passed" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr


def test_python_abi_tests_under_sanitizers(sanitized):
    env = _env(sanitized["rt"])
    env["LD_PRELOAD"] = sanitized["rt"]
    env["AB_ATTN_LIBRARY"] = sanitized["lib"]
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         capture_output=True, text=True, timeout=900, env=env, cwd=ROOT)
    assert res.returncode == 0, (res.stdout[-3000:], res.stderr[-3000:])
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr
