"""The C-ABI library: it loads, exports every entry point its header declares,
and rejects bad arguments on the host before touching the device. None of these
calls launch GPU work, so they run without a GPU."""
import ctypes
import os
import re
import struct

import numpy as np
import pytest

import resumable_checkpoint_state_amd as rcs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rcs.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(rcs.LIB_PATH):
        rcs.build()
    return rcs.lib()


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ["adamw_clip_step", "grad_global_norm", "ckpt_pack", "ckpt_unpack",
                     "ckpt_bytes", "last_grad_norm", "rcs_strerror"]:
        assert required in names


def test_library_exports_every_declared_symbol(L):
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_library_is_built_for_gfx950():
    data = open(rcs.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def test_ckpt_bytes_closed_form(L):
    for n in [1, 3, 262_144, 12_800_000, 124_356_864, 2_000_000_000, 2**31 - 1]:
        assert rcs.ckpt_bytes(n) == 8 + 12 * n
    for n in [0, -5, 2**31]:
        assert rcs.ckpt_bytes(n) == -1


def test_strerror_covers_codes(L):
    for code in [rcs.OK, rcs.EINVAL, rcs.ESIZE, rcs.EHEADER, rcs.EHIP, rcs.ENOMEM]:
        assert rcs.strerror(code) and rcs.strerror(code) != "unknown status"


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: rejected before any device check


@pytest.mark.parametrize("n,t,lr,wd,clip", [
    (0, 1, 1e-3, 0.0, 1.0), (-1, 1, 1e-3, 0.0, 1.0), (2**31, 1, 1e-3, 0.0, 1.0),
    (16, 0, 1e-3, 0.0, 1.0), (16, -3, 1e-3, 0.0, 1.0), (16, 1, float("nan"), 0.0, 1.0),
    (16, 1, float("inf"), 0.0, 1.0), (16, 1, 1e-3, float("nan"), 1.0),
    (16, 1, 1e-3, 0.0, 0.0), (16, 1, 1e-3, 0.0, -1.0), (16, 1, 1e-3, 0.0, float("nan")),
])
def test_adamw_clip_step_rejects_bad_scalars(L, n, t, lr, wd, clip):
    rc = L.adamw_clip_step(FAKE, FAKE, FAKE, FAKE, n, t, lr, wd, clip, None)
    assert rc == rcs.EINVAL
    rc = L.adamw_clip_step_noalloc(FAKE, FAKE, FAKE, FAKE, n, t, lr, wd, clip, None, None)
    assert rc == rcs.EINVAL


def test_null_pointers_rejected(L):
    assert L.adamw_clip_step(None, None, None, None, 16, 1, 1e-3, 0.0, 1.0, None) == rcs.EINVAL
    assert L.grad_global_norm(None, 16, None, None) == rcs.EINVAL
    assert L.grad_zero(None, 16, None) == rcs.EINVAL
    assert L.grad_zero(FAKE, 0, None) == rcs.EINVAL
    assert L.grad_zero(FAKE, 2**31, None) == rcs.EINVAL
    assert L.last_grad_norm(None, None) == rcs.EINVAL
    buf = (ctypes.c_uint8 * 20)()
    assert L.ckpt_pack(1, 1, FAKE, FAKE, FAKE, None, 20, None) == rcs.EINVAL
    assert L.ckpt_pack(-1, 1, FAKE, FAKE, FAKE, buf, 20, None) == rcs.EINVAL
    assert L.ckpt_pack(1, 1, FAKE, FAKE, FAKE, buf, 19, None) == rcs.ESIZE
    step = ctypes.c_int32(-7)
    assert L.ckpt_unpack(None, 20, 1, ctypes.byref(step), FAKE, FAKE, FAKE, None) == rcs.EINVAL
    assert L.ckpt_unpack(buf, 20, 1, None, FAKE, FAKE, FAKE, None) == rcs.EINVAL
    assert L.ckpt_unpack(buf, 20, 0, ctypes.byref(step), FAKE, FAKE, FAKE, None) == rcs.EINVAL


def _packed(step, n):
    return bytearray(struct.pack("<ii", step, n) + bytes(12 * n))


@pytest.mark.parametrize("case,want", [
    ("short_header", rcs.ESIZE), ("truncated", rcs.ESIZE), ("extended", rcs.ESIZE),
    ("n_zero", rcs.EHEADER), ("n_negative", rcs.EHEADER), ("n_mismatch", rcs.EHEADER),
    ("step_negative", rcs.EHEADER),
])
def test_unpack_header_faults_rejected_before_any_copy(L, case, want):
    """Fault injection on the host: every malformed buffer is rejected by the
    header checks, which run before any device pointer is looked at, and the
    step output is left untouched."""
    n = 16
    b = _packed(5, n)
    if case == "short_header":
        b = b[:7]
    elif case == "truncated":
        b = b[:-1]
    elif case == "extended":
        b = b + b"\0"
    elif case == "n_zero":
        b[4:8] = struct.pack("<i", 0)
    elif case == "n_negative":
        b[4:8] = struct.pack("<i", -n)
    elif case == "n_mismatch":
        b[4:8] = struct.pack("<i", n + 1)
    elif case == "step_negative":
        b[0:4] = struct.pack("<i", -1)
    arr = (ctypes.c_uint8 * len(b)).from_buffer(b)
    step = ctypes.c_int32(-7)
    rc = L.ckpt_unpack(arr, len(b), n, ctypes.byref(step), FAKE, FAKE, FAKE, None)
    assert rc == want
    assert step.value == -7


def test_writer_argument_rejections_need_no_device(L):
    import ctypes
    h = ctypes.c_void_p()
    assert L.rcs_ckpt_writer_create(None, 10, 1, ctypes.byref(h)) == rcs.EINVAL
    assert L.rcs_ckpt_writer_create(b"/tmp", 0, 1, ctypes.byref(h)) == rcs.EINVAL
    assert L.rcs_ckpt_writer_create(b"/tmp", rcs.MAX_N + 1, 1, ctypes.byref(h)) == rcs.EINVAL
    assert L.rcs_ckpt_writer_create(b"/tmp", 10, 0, ctypes.byref(h)) == rcs.EINVAL
    assert L.rcs_ckpt_writer_create(b"/tmp", 10, 1, None) == rcs.EINVAL
    assert L.rcs_ckpt_writer_submit(None, 1, None, None, None, None) == rcs.EINVAL
    assert L.rcs_ckpt_writer_wait(None, None, 0) == rcs.EINVAL
    assert L.rcs_ckpt_writer_destroy(None) == rcs.OK


def test_python_binding_rejects_host_tensors():
    import torch
    a = torch.zeros(8)
    with pytest.raises(TypeError):
        rcs.adamw_clip_step(a, a, a, a, 1, 1e-3, 0.0, 1.0)
    with pytest.raises(TypeError):
        rcs.grad_global_norm(a)


def test_step_file_name():
    assert rcs.step_file_name(80) == "step_000080.bin"
    assert rcs.step_file_name(112700) == "step_112700.bin"
    assert rcs.step_file_name(1234567) == "step_1234567.bin"


def test_missing_library_fails_loudly(monkeypatch):
    """No CPU fallback: without librcs.so every entry point raises."""
    monkeypatch.setattr(rcs, "LIB_PATH", "/nonexistent/librcs.so")
    monkeypatch.setattr(rcs, "_lib", None)
    with pytest.raises(ImportError):
        rcs.lib()
    with pytest.raises(ImportError):
        rcs.ckpt_bytes(10)


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_unpack_header_decisions_match_the_oracle_on_random_buffers(L):
    """2,000 seeded random step-file images (steps and sizes around the
    edges: negative, zero, the expected n and its neighbours, int32 extremes;
    lengths exact, one byte off, short of the header) through the library's
    and the oracle's unpack: the same status for every rejected image (the
    library's checks run before any device pointer is looked at, and leave
    the step output untouched), and for every image the oracle accepts the
    library passes the header checks too (it then refuses the stand-in device
    pointers with RCS_EINVAL, having copied nothing)."""
    import numpy as np
    import oracle

    rng = np.random.default_rng(20240611)
    steps = [-(2**31), -5, -1, 0, 1, 7, 112_700, 2**31 - 1]
    seen = {oracle.OK: 0, oracle.ESIZE: 0, oracle.EHEADER: 0}
    for case in range(2000):
        n_exp = int(rng.integers(1, 65))
        step = int(rng.choice(steps))
        n_hdr = int(rng.choice([n_exp, n_exp, n_exp - 1, n_exp + 1, 0, -n_exp, 2**31 - 1,
                                -(2**31), int(rng.integers(1, 200))]))
        body = 12 * n_hdr if 0 < n_hdr <= 64 else 12 * n_exp
        length = int(rng.choice([8 + body, 8 + body, 8 + body - 1, 8 + body + 1,
                                 int(rng.integers(0, 8)), 8 + 12 * n_exp]))
        full = struct.pack("<ii", step, n_hdr) + rng.integers(0, 256, body + 16,
                                                             dtype=np.uint8).tobytes()
        b = bytearray(full[:length]) if length > 0 else bytearray(1)
        w, m, v = (np.zeros(n_exp, np.float32) for _ in range(3))
        orc, _ = oracle.ckpt_unpack(np.frombuffer(bytes(b[:length]), np.uint8).copy()
                                    if length > 0 else np.zeros(0, np.uint8), w, m, v)
        arr = (ctypes.c_uint8 * len(b)).from_buffer(b)
        out = ctypes.c_int32(-7)
        rc = L.ckpt_unpack(arr, length, n_exp, ctypes.byref(out), FAKE, FAKE, FAKE, None)
        ctx = (case, step, n_hdr, n_exp, length)
        if orc == oracle.OK:
            assert rc == rcs.EINVAL, ctx
        else:
            assert rc == orc, ctx
        assert out.value == -7, ctx
        seen[orc] += 1
    assert min(seen.values()) > 100, seen


def test_ceilings_library_loads_and_rejects_bad_arguments():
    """bench.py's streaming-ceiling library: built for gfx950, exports its two
    calls, and refuses bad arguments before any HIP call (no GPU needed)."""
    path = os.path.join(ROOT, "resumable_checkpoint_state_amd", "libceilings.so")
    if not os.path.exists(path):
        from resumable_checkpoint_state_amd import _build
        _build.build_ceilings()
    assert b"gfx950" in open(path, "rb").read()
    C = ctypes.CDLL(path)
    C.rcs_ceiling_blocks.argtypes = [ctypes.c_int64]
    C.rcs_ceiling_blocks.restype = ctypes.c_int64
    vp = ctypes.c_void_p
    C.rcs_ceiling_time.argtypes = [ctypes.c_int, vp, vp, vp, vp, ctypes.c_int64, vp,
                                   ctypes.c_int, vp, ctypes.POINTER(ctypes.c_double)]
    C.rcs_ceiling_time.restype = ctypes.c_int
    # the read's grid: one block per 2048 vectors, at most 256
    assert [C.rcs_ceiling_blocks(k) for k in (0, 1, 2048, 2049, 1 << 30)] == [0, 1, 1, 2, 256]
    us = ctypes.c_double(-1.0)
    fake = 0x1000
    bad = [(4, fake, fake, fake, fake, 16, fake, 10),   # no such kind
           (-1, fake, fake, fake, fake, 16, fake, 10),
           (2, fake, fake, fake, fake, 0, fake, 10),    # no vectors
           (2, fake, fake, fake, fake, 16, fake, 0),    # no launches
           (2, fake, fake, fake, fake, 16, fake, 1001),
           (0, fake, fake + 4, fake, fake, 16, fake, 10),  # g off a 16-byte boundary
           (0, fake, fake, fake, fake, 16, None, 10),   # no output for the read
           (1, None, fake, fake, fake, 16, fake, 10),
           (2, fake, fake, fake, fake + 8, 16, fake, 10)]
    for args in bad:
        assert C.rcs_ceiling_time(*args, None, ctypes.byref(us)) == -1, args
    assert C.rcs_ceiling_time(2, fake, fake, fake, fake, 16, fake, 10, None, None) == -1
    assert us.value == -1.0
