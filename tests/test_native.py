"""Native callers of the library, built with the host compilers:
include/rcs.h compiles as C and a C program links and calls librcs.so (host
rejections here; a whole C training loop with pack, file write and the
asynchronous writer on the GPU, checked against the oracle); the host
file-IO code runs under AddressSanitizer and UndefinedBehaviorSanitizer, the
asynchronous writer under ThreadSanitizer (host code only: no device code is
built with a sanitizer)."""
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


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")
def test_async_writer_under_thread_sanitizer(tmp_path):
    """The asynchronous writer's worker thread, lock and condition variable
    under ThreadSanitizer, with concurrent submit and wait calls; the device
    side is a host stand-in (tests/native/writer_tsan_driver.cpp), the file
    side the real ckpt_io.cpp."""
    exe = tmp_path / "writer_tsan_driver"
    csrc = os.path.join(ROOT, "resumable_checkpoint_state_amd", "csrc")
    _run(["g++", "-std=c++17", "-g", "-O1", "-fsanitize=thread", *HIP_DEFS, f"-I{csrc}",
          os.path.join(csrc, "ckpt_writer.cpp"), os.path.join(csrc, "ckpt_io.cpp"),
          os.path.join(NATIVE, "writer_tsan_driver.cpp"), "-o", str(exe), "-lpthread"])
    d = tmp_path / "files"
    d.mkdir()
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1")
    assert "writer tsan driver ok" in _run([str(exe), str(d)], env=env)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "oracle_driver"
    _run(["gcc", "-std=c11", "-g", "-O1", "-ffp-contract=off", "-fno-fast-math",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(NATIVE, "oracle_driver.c"),
          "-lm", "-o", str(exe)])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0")
    assert "oracle driver ok" in _run([str(exe)], env=env)


@pytest.mark.gpu
@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
@pytest.mark.parametrize("n", [100_003, 5_000_001])
def test_c_program_trains_and_saves_on_the_gpu(tmp_path, n):
    """A C program drives three updates, the pack, the step-file write and the
    asynchronous writer through the C ABI alone; its norms and its file match
    the oracle run on the same inputs (one and several grid-stride passes of
    the norm kernel; both sizes have a ragged tail)."""
    import numpy as np

    import oracle
    import workloads
    from util import max_ulp

    exe = tmp_path / "c_step_driver"
    libdir = os.path.dirname(rcs.LIB_PATH)
    _run(["gcc", "-std=c11", "-Wall", "-Werror", *HIP_DEFS, os.path.join(NATIVE, "c_step_driver.c"),
          f"-L{libdir}", "-l:librcs.so", f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{libdir}",
          f"-Wl,-rpath,{ROCM}/lib", "-o", str(exe)])
    steps, lr, wd, clip = 3, 3e-3, 0.01, 1.0
    w0 = workloads.custom(310, n, 0.02).numpy()
    gs = [workloads.custom(311 + t, n, sigma).numpy() for t, sigma in enumerate((1e-3, 1e-2, 2e-3))]
    inp = tmp_path / "in.bin"
    with open(inp, "wb") as f:
        for a in (w0, *gs):
            f.write(a.astype("<f4").tobytes())
    d1, d2 = tmp_path / "file", tmp_path / "writer"
    d1.mkdir()
    d2.mkdir()
    out = _run([str(exe), str(inp), str(n), str(steps), repr(lr), repr(wd), repr(clip), str(d1),
                str(d2)], timeout=120)
    assert "c step driver ok" in out
    norms, paths = {}, {}
    for ln in out.splitlines():
        key, _, rest = ln.partition(" ")
        if key == "norm":
            t, x = rest.split()
            norms[int(t)] = float(x)
        elif key in ("file", "writer"):
            paths[key] = rest
    ow, om, ov = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in range(1, steps + 1):
        rc, on = oracle.adamw_clip_step(ow, gs[t - 1], om, ov, t, lr, wd, clip)
        assert rc == oracle.OK
        gn = norms[t]
        assert abs(gn - on) <= 1e-12 * on, (t, gn, on)
    raw = open(paths["file"], "rb").read()
    assert os.path.basename(paths["file"]) == "step_000003.bin"
    _, expect = oracle.ckpt_pack(steps, ow, om, ov)
    assert raw[:8] == expect.tobytes()[:8]
    got = np.frombuffer(raw, dtype=np.uint8)
    for j, ref in enumerate((ow, om, ov)):
        arr = got[8 + 4 * j * n: 8 + 4 * (j + 1) * n].view(np.float32)
        assert max_ulp(arr, ref) <= 2, j
    assert os.path.basename(paths["writer"]) == "step_000003.bin"
    assert open(paths["writer"], "rb").read() == raw


@pytest.mark.gpu
def test_c_abi_refuses_exact_size_short_buffers(tmp_path):
    """hipMalloc'd arrays of exactly their own size, one of them shorter than
    n: every call that takes device arrays returns RCS_ESIZE and nothing is
    launched (the arrays keep a byte pattern any kernel or copy would
    overwrite)."""
    exe = tmp_path / "abi_short_buffers"
    libdir = os.path.dirname(rcs.LIB_PATH)
    _run(["gcc", "-std=c11", "-Wall", "-Werror", *HIP_DEFS,
          os.path.join(NATIVE, "abi_short_buffers.c"), f"-L{libdir}", "-l:librcs.so",
          f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{ROCM}/lib",
          "-o", str(exe)])
    assert "abi short buffers ok" in _run([str(exe)], timeout=120)
