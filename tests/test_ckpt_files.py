"""On-disk step files and the SIGTERM/SIGUSR1 flags: host-only parts of the
library, run without a GPU. Packed buffers come from the oracle's pack, so
the files are checked against an independent writer of the layout."""
import os
import signal
import struct

import numpy as np
import pytest
import torch

import oracle
import resumable_checkpoint_state_amd as rcs


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(rcs.LIB_PATH):
        rcs.build()
    rcs.lib()


def packed(step, n, seed=0):
    rng = np.random.default_rng(seed)
    w, m, v = (rng.standard_normal(n).astype(np.float32) for _ in range(3))
    rc, buf = oracle.ckpt_pack(step, w, m, v)
    assert rc == oracle.OK
    return torch.from_numpy(buf)


def test_atomic_write_bytes_exact(tmp_path):
    buf = packed(80, 1001)
    path = rcs.ckpt_file_write(tmp_path, buf)
    assert os.path.basename(path) == "step_000080.bin"
    assert sorted(os.listdir(tmp_path)) == ["step_000080.bin"]  # no temporary left
    assert open(path, "rb").read() == buf.numpy().tobytes()
    back = rcs.ckpt_file_read(path, pin=False)
    assert torch.equal(back, buf)


def test_write_rejects_inconsistent_buffers(tmp_path):
    buf = packed(3, 10)
    with pytest.raises(rcs.RcsError) as e:
        rcs.ckpt_file_write(tmp_path, buf[:-1].clone())
    assert e.value.status == rcs.ESIZE
    bad = buf.clone()
    bad[0:4] = torch.from_numpy(np.frombuffer(struct.pack("<i", -2), np.uint8).copy())
    with pytest.raises(rcs.RcsError) as e:
        rcs.ckpt_file_write(tmp_path, bad)
    assert e.value.status == rcs.EHEADER
    assert os.listdir(tmp_path) == []


def test_read_rejects_wrong_size_and_header(tmp_path):
    path = rcs.ckpt_file_write(tmp_path, packed(5, 16))
    with pytest.raises(rcs.RcsError) as e:
        rcs.ckpt_file_read(path, buf=torch.empty(8 + 12 * 16 + 1, dtype=torch.uint8))
    assert e.value.status == rcs.ESIZE
    raw = bytearray(open(path, "rb").read())
    raw[4:8] = struct.pack("<i", 15)
    open(path, "wb").write(raw)
    with pytest.raises(rcs.RcsError) as e:
        rcs.ckpt_file_read(path, pin=False)
    assert e.value.status in (rcs.ESIZE, rcs.EHEADER)
    with pytest.raises(rcs.RcsError) as e:
        rcs.ckpt_file_read(tmp_path / "step_999999.bin", pin=False)
    assert e.value.status == rcs.ENOENT


def test_latest_skips_partial_and_malformed_files(tmp_path):
    assert rcs.ckpt_file_latest(tmp_path) is None
    for s in (100, 200, 300):
        rcs.ckpt_file_write(tmp_path, packed(s, 64, seed=s))
    # a crash mid-write leaves only a temporary: never picked
    open(tmp_path / "step_000400.bin.tmp", "wb").write(packed(400, 64).numpy().tobytes())
    # a truncated file with a newer name: rejected by the size check
    open(tmp_path / "step_000500.bin", "wb").write(packed(500, 64).numpy().tobytes()[:-3])
    # header step that disagrees with the name
    open(tmp_path / "step_000600.bin", "wb").write(packed(7, 64).numpy().tobytes())
    # unrelated names
    open(tmp_path / "step_abc.bin", "wb").write(b"xx")
    open(tmp_path / "notes.txt", "wb").write(b"yy")
    step, path = rcs.ckpt_file_latest(tmp_path)
    assert step == 300 and os.path.basename(path) == "step_000300.bin"


def test_rotation_keeps_newest_and_clears_temporaries(tmp_path):
    for s in (1, 2, 3, 4, 5, 6):
        rcs.ckpt_file_write(tmp_path, packed(s, 8, seed=s))
    open(tmp_path / "step_000007.bin.tmp", "wb").write(b"partial")
    removed = rcs.ckpt_file_rotate(tmp_path, 3)
    assert removed == 4
    assert sorted(os.listdir(tmp_path)) == ["step_000004.bin", "step_000005.bin",
                                            "step_000006.bin"]


def test_wide_step_numbers(tmp_path):
    path = rcs.ckpt_file_write(tmp_path, packed(1234567, 4))
    assert os.path.basename(path) == "step_1234567.bin"
    rcs.ckpt_file_write(tmp_path, packed(999999, 4))
    assert rcs.ckpt_file_latest(tmp_path)[0] == 1234567


def test_signal_flags_are_polled_and_cleared():
    rcs.signals_install()
    try:
        assert rcs.signals_poll() == 0
        os.kill(os.getpid(), signal.SIGUSR1)
        assert rcs.signals_poll() == rcs.SIG_WRITE_CONTINUE
        assert rcs.signals_poll() == 0
        os.kill(os.getpid(), signal.SIGTERM)
        assert rcs.signals_poll() == rcs.SIG_WRITE_EXIT
        os.kill(os.getpid(), signal.SIGUSR1)
        os.kill(os.getpid(), signal.SIGTERM)
        assert rcs.signals_poll() == rcs.SIG_WRITE_CONTINUE | rcs.SIG_WRITE_EXIT
        assert rcs.signals_poll() == 0
    finally:
        signal.signal(signal.SIGTERM, signal.SIG_DFL)
        signal.signal(signal.SIGUSR1, signal.SIG_DFL)


def test_short_path_buffer_refused_before_writing(tmp_path):
    """ckpt_file_write with a path_out too small for the final path returns
    RCS_EINVAL and leaves the directory as it was (through the C ABI)."""
    import ctypes
    buf = packed(7, 12)
    small = ctypes.create_string_buffer(8)
    rc = rcs.lib().ckpt_file_write(os.fsencode(str(tmp_path)), ctypes.c_void_p(buf.data_ptr()),
                                   buf.numel(), small, 8)
    assert rc == rcs.EINVAL
    assert os.listdir(tmp_path) == []
