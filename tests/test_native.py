"""Native callers of the library, built here with the host compilers:
include/rcs.h compiles as C and a C program links and calls librcs.so; the
host file-IO code runs under AddressSanitizer and UndefinedBehaviorSanitizer
(host code only: no device code is built with a sanitizer)."""
import os
import shutil
import subprocess

import pytest

import resumable_checkpoint_state_amd as rcs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIP_DEFS = ["-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include"]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(rcs.LIB_PATH):
        rcs.build()


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_c_caller_compiles_links_and_runs(tmp_path):
    exe = tmp_path / "abi_c_caller"
    libdir = os.path.dirname(rcs.LIB_PATH)
    _run(["gcc", "-std=c11", "-Wall", "-Werror", *HIP_DEFS, os.path.join(NATIVE, "abi_c_caller.c"),
          f"-L{libdir}", "-l:librcs.so", f"-Wl,-rpath,{libdir}", "-o", str(exe)])
    assert "c caller ok" in _run([str(exe)])


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")
def test_file_io_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "ckpt_io_driver"
    src = os.path.join(ROOT, "resumable_checkpoint_state_amd", "csrc", "ckpt_io.cpp")
    _run(["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", *HIP_DEFS, src,
          os.path.join(NATIVE, "ckpt_io_driver.cpp"), "-o", str(exe)])
    d = tmp_path / "files"
    d.mkdir()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0")
    assert "ckpt_io driver ok" in _run([str(exe), str(d)], env=env)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "oracle_driver"
    _run(["gcc", "-std=c11", "-g", "-O1", "-ffp-contract=off", "-fno-fast-math",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(NATIVE, "oracle_driver.c"),
          "-lm", "-o", str(exe)])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0")
    assert "oracle driver ok" in _run([str(exe)], env=env)
