"""Thin Python binding of librcs.so (the gfx950 clip+AdamW / step-file library).

Argument marshalling only: every step of the update runs in the HIP kernels of
csrc/rcs.hip behind the C ABI declared in include/rcs.h. PyTorch supplies the
device memory (CUDA tensors on ROCm) and the stream
(``torch.cuda.current_stream().cuda_stream`` is the HIP stream handle).

There is no fallback: if librcs.so is missing or cannot be loaded, every call
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

from ._build import LIB as LIB_PATH
from ._build import build

__all__ = [
    "RcsError", "adamw_clip_step", "adamw_clip_step_noalloc", "adamw_clip_step_accum",
    "grad_clip_inplace", "grad_zero", "grad_global_norm", "last_grad_norm", "ckpt_bytes",
    "ckpt_pack", "ckpt_unpack", "init", "profile_enable", "profile_read",
    "strerror", "lib", "LIB_PATH", "build", "step_file_name", "MAX_N",
    "ckpt_pack_async", "ckpt_pack_wait", "CkptWriter", "StepFileCheckpointer",
]

OK, EINVAL, ESIZE, EHEADER, EHIP, ENOMEM, EIO, ENOENT = 0, -1, -2, -3, -4, -5, -6, -7
SIG_WRITE_CONTINUE, SIG_WRITE_EXIT = 1, 2
MAX_N = 2_147_483_647


class RcsError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


_lib: ctypes.CDLL | None = None


def lib() -> ctypes.CDLL:
    """Loads librcs.so (built in-tree by build()); raises if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python -m resumable_checkpoint_state_amd._build")
    L = ctypes.CDLL(LIB_PATH)
    vp, f32p = ctypes.c_void_p, ctypes.c_void_p
    i64, i32, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    L.rcs_strerror.argtypes = [ctypes.c_int]
    L.rcs_strerror.restype = ctypes.c_char_p
    L.rcs_init.argtypes = [ctypes.c_int, vp]
    L.rcs_init.restype = ctypes.c_int
    L.adamw_clip_step.argtypes = [f32p, f32p, f32p, f32p, i64, i32, f32, f32, f32, vp]
    L.adamw_clip_step.restype = ctypes.c_int
    L.grad_global_norm.argtypes = [f32p, i64, vp, vp]
    L.grad_global_norm.restype = ctypes.c_int
    L.last_grad_norm.argtypes = [vp, vp]
    L.last_grad_norm.restype = ctypes.c_int
    L.ckpt_bytes.argtypes = [i64]
    L.ckpt_bytes.restype = i64
    L.ckpt_pack.argtypes = [i32, i64, f32p, f32p, f32p, vp, i64, vp]
    L.ckpt_pack.restype = ctypes.c_int
    L.ckpt_unpack.argtypes = [vp, i64, i64, ctypes.POINTER(i32), f32p, f32p, f32p, vp]
    L.ckpt_unpack.restype = ctypes.c_int
    L.rcs_profile_enable.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    L.rcs_profile_enable.restype = ctypes.c_int
    L.rcs_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double),
                                   ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
    L.rcs_profile_read.restype = ctypes.c_int
    L.adamw_clip_step_noalloc.argtypes = [f32p, f32p, f32p, f32p, i64, i32, f32, f32, f32, vp,
                                          vp]
    L.adamw_clip_step_noalloc.restype = ctypes.c_int
    L.adamw_clip_step_accum.argtypes = [f32p, f32p, f32p, f32p, i64, i32, f32, f32, f32, f32, vp]
    L.adamw_clip_step_accum.restype = ctypes.c_int
    L.grad_clip_inplace.argtypes = [f32p, i64, f32, vp]
    L.grad_clip_inplace.restype = ctypes.c_int
    L.grad_zero.argtypes = [f32p, i64, vp]
    L.grad_zero.restype = ctypes.c_int
    L.ckpt_snapshot_bytes.argtypes = [i64]
    L.ckpt_snapshot_bytes.restype = i64
    L.ckpt_pack_async.argtypes = [i32, i64, f32p, f32p, f32p, f32p, i64, vp, i64, vp, vp]
    L.ckpt_pack_async.restype = ctypes.c_int
    L.ckpt_pack_wait.argtypes = [f32p]
    L.ckpt_pack_wait.restype = ctypes.c_int
    cp = ctypes.c_char_p
    L.ckpt_file_write.argtypes = [cp, vp, i64, ctypes.c_char_p, i64]
    L.ckpt_file_write.restype = ctypes.c_int
    L.ckpt_file_write_path.argtypes = [cp, vp, i64]
    L.ckpt_file_write_path.restype = ctypes.c_int
    L.rcs_file_write_atomic.argtypes = [cp, vp, i64]
    L.rcs_file_write_atomic.restype = ctypes.c_int
    L.ckpt_file_size.argtypes = [cp]
    L.ckpt_file_size.restype = i64
    L.ckpt_file_read.argtypes = [cp, vp, i64]
    L.ckpt_file_read.restype = ctypes.c_int
    L.ckpt_file_latest.argtypes = [cp, ctypes.POINTER(i32), ctypes.c_char_p, i64]
    L.ckpt_file_latest.restype = ctypes.c_int
    L.ckpt_file_rotate.argtypes = [cp, ctypes.c_int]
    L.ckpt_file_rotate.restype = ctypes.c_int
    L.rcs_signals_install.argtypes = []
    L.rcs_signals_install.restype = ctypes.c_int
    L.rcs_signals_poll.argtypes = []
    L.rcs_signals_poll.restype = ctypes.c_int
    L.rcs_ckpt_writer_create.argtypes = [cp, i64, ctypes.c_int, ctypes.POINTER(vp)]
    L.rcs_ckpt_writer_create.restype = ctypes.c_int
    L.rcs_ckpt_writer_submit.argtypes = [vp, i32, f32p, f32p, f32p, vp]
    L.rcs_ckpt_writer_submit.restype = ctypes.c_int
    L.rcs_ckpt_writer_wait.argtypes = [vp, ctypes.c_char_p, i64]
    L.rcs_ckpt_writer_wait.restype = ctypes.c_int
    L.rcs_ckpt_writer_destroy.argtypes = [vp]
    L.rcs_ckpt_writer_destroy.restype = ctypes.c_int
    _lib = L
    return L


def strerror(status: int) -> str:
    return lib().rcs_strerror(status).decode()


def _check(rc: int, where: str) -> int:
    if rc < 0:
        raise RcsError(rc, where)
    return rc


# The current stream's raw handle without building a torch.cuda.Stream object
# (a few microseconds per call, which matters for small updates).
_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, device: int | None = None) -> int:
    if stream is None:
        if _raw_current_stream is not None:
            return _raw_current_stream(torch.cuda.current_device() if device is None else device)
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev_f32(t: torch.Tensor, name: str, n: int | None = None, cur: int | None = None) -> int:
    """Device pointer of a contiguous float32 tensor on the current device
    (cur: the current device index, when the caller already has it)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != torch.float32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous float32 tensor")
    if n is not None and t.numel() != n:
        raise ValueError(f"{name} has {t.numel()} elements, expected {n}")
    if cur is None:
        cur = torch.cuda.current_device()
    if t.get_device() != cur:
        raise ValueError(f"{name} is on {t.device}; the library works on the current device "
                         f"(cuda:{cur}): use torch.cuda.device(...)")
    return t.data_ptr()


def init(device: int | None = None, stream=None) -> None:
    """Allocates the (device, stream) workspace ahead of the first step."""
    dev = torch.cuda.current_device() if device is None else device
    _check(lib().rcs_init(dev, _stream(stream)), "rcs_init")


def adamw_clip_step(w, g, m, v, t: int, lr: float, wd: float, clip: float, stream=None) -> None:
    """One clipped AdamW update of w, m, v in place (asynchronous on stream)."""
    n, wp = w.numel(), _dev_f32(w, "w")
    cur = w.get_device()  # the current device, checked just above
    args = (wp, _dev_f32(g, "g", n, cur), _dev_f32(m, "m", n, cur), _dev_f32(v, "v", n, cur))
    _check(lib().adamw_clip_step(*args, n, int(t), float(lr), float(wd), float(clip),
                                 _stream(stream, cur)), "adamw_clip_step")


def adamw_clip_step_noalloc(w, g, m, v, t: int, lr: float, wd: float, clip: float,
                            norm_out: torch.Tensor | None = None, stream=None) -> None:
    """adamw_clip_step without any allocation: the norm buffers are the
    library's static device array (shared by every call on the GPU, so calls
    must not overlap on the device). norm_out: optional 1-element float64
    device or pinned host tensor that receives the pre-clip norm."""
    n, wp = w.numel(), _dev_f32(w, "w")
    cur = w.get_device()
    args = (wp, _dev_f32(g, "g", n, cur), _dev_f32(m, "m", n, cur), _dev_f32(v, "v", n, cur))
    np_ = None if norm_out is None else _norm_out(norm_out).data_ptr()
    _check(lib().adamw_clip_step_noalloc(*args, n, int(t), float(lr), float(wd), float(clip),
                                         np_, _stream(stream, cur)), "adamw_clip_step_noalloc")


def adamw_clip_step_accum(w, g_sum, m, v, t: int, lr: float, wd: float, clip: float,
                          grad_scale: float, stream=None) -> None:
    """The update for a gradient summed over micro-batches: each element of
    g_sum is multiplied by the float32 grad_scale (1/n_micro) inside the
    kernels before norm, clip and update; g_sum is not written."""
    n, wp = w.numel(), _dev_f32(w, "w")
    cur = w.get_device()
    args = (wp, _dev_f32(g_sum, "g", n, cur), _dev_f32(m, "m", n, cur), _dev_f32(v, "v", n, cur))
    _check(lib().adamw_clip_step_accum(*args, n, int(t), float(lr), float(wd), float(clip),
                                       float(grad_scale), _stream(stream, cur)),
           "adamw_clip_step_accum")


def grad_clip_inplace(g, clip: float, stream=None) -> None:
    """g *= clip/||g|| in place when ||g|| > clip (the global clip on its own)."""
    _check(lib().grad_clip_inplace(_dev_f32(g, "g"), g.numel(), float(clip), _stream(stream)),
           "grad_clip_inplace")


def grad_zero(g, stream=None) -> None:
    """g = 0 in place: clears the accumulation buffer after the step."""
    _check(lib().grad_zero(_dev_f32(g, "g"), g.numel(), _stream(stream)), "grad_zero")


def _norm_out(out):
    if out is None:
        out = torch.empty(1, dtype=torch.float64, device="cuda")
    if out.dtype != torch.float64 or out.numel() < 1 or not out.is_contiguous():
        raise TypeError("norm output must be a contiguous float64 tensor")
    if not out.is_cuda and not out.is_pinned():
        raise TypeError("norm output must be device or pinned host memory")
    return out


def grad_global_norm(g, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Pre-clip global L2 norm of g into a 1-element float64 tensor."""
    gp = _dev_f32(g, "g")
    out = _norm_out(out)
    _check(lib().grad_global_norm(gp, g.numel(), out.data_ptr(), _stream(stream)),
           "grad_global_norm")
    return out


def last_grad_norm(out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The pre-clip norm of the last update enqueued on the stream."""
    out = _norm_out(out)
    _check(lib().last_grad_norm(_stream(stream), out.data_ptr()), "last_grad_norm")
    return out


def ckpt_bytes(n: int) -> int:
    return lib().ckpt_bytes(n)


def step_file_name(step: int) -> str:
    """step_NNNNNN.bin, six digits, widening past 999,999."""
    return "step_%06d.bin" % step


def _host_u8(buf: torch.Tensor, name: str) -> int:
    if not isinstance(buf, torch.Tensor) or buf.is_cuda or buf.dtype != torch.uint8 \
            or not buf.is_contiguous():
        raise TypeError(f"{name} must be a contiguous uint8 host tensor (pinned for async copies)")
    return buf.data_ptr()


def ckpt_pack(step: int, w, m, v, buf: torch.Tensor, stream=None) -> torch.Tensor:
    """Packs [int32 step][int32 n][w][m][v] into the host tensor buf."""
    n = w.numel()
    ptrs = (_dev_f32(w, "w"), _dev_f32(m, "m", n), _dev_f32(v, "v", n))
    _check(lib().ckpt_pack(int(step), n, *ptrs, _host_u8(buf, "buf"), buf.numel(),
                           _stream(stream)), "ckpt_pack")
    return buf


def ckpt_unpack(buf: torch.Tensor, w, m, v, stream=None) -> int:
    """Validates buf and copies its arrays into w, m, v; returns the header step."""
    n = w.numel()
    ptrs = (_dev_f32(w, "w"), _dev_f32(m, "m", n), _dev_f32(v, "v", n))
    step = ctypes.c_int32(-1)
    _check(lib().ckpt_unpack(_host_u8(buf, "buf"), buf.numel(), n, ctypes.byref(step), *ptrs,
                             _stream(stream)), "ckpt_unpack")
    return step.value


def ckpt_snapshot_bytes(n: int) -> int:
    return lib().ckpt_snapshot_bytes(n)


def ckpt_pack_async(step: int, w, m, v, snapshot, buf: torch.Tensor, compute_stream=None,
                    copy_stream=None) -> torch.Tensor:
    """Snapshot w, m, v on the compute stream, drain to buf on the copy stream;
    call ckpt_pack_wait(snapshot) before reading buf."""
    n = w.numel()
    ptrs = (_dev_f32(w, "w"), _dev_f32(m, "m", n), _dev_f32(v, "v", n))
    sp = _dev_f32(snapshot, "snapshot", 3 * n)
    if copy_stream is None:
        raise ValueError("ckpt_pack_async needs a separate copy stream")
    _check(lib().ckpt_pack_async(int(step), n, *ptrs, sp, 4 * snapshot.numel(),
                                 _host_u8(buf, "buf"), buf.numel(), _stream(compute_stream),
                                 _stream(copy_stream)), "ckpt_pack_async")
    return buf


def ckpt_pack_wait(snapshot) -> None:
    _check(lib().ckpt_pack_wait(_dev_f32(snapshot, "snapshot")), "ckpt_pack_wait")


def _b(path) -> bytes:
    return os.fsencode(path)


def ckpt_file_write(directory, buf: torch.Tensor) -> str:
    """Atomically writes a packed state (copies complete) as <dir>/step_NNNNNN.bin."""
    out = ctypes.create_string_buffer(4096)
    _check(lib().ckpt_file_write(_b(directory), _host_u8(buf, "buf"), buf.numel(), out, 4096),
           "ckpt_file_write")
    return os.fsdecode(out.value)


def ckpt_file_read(path, buf: torch.Tensor | None = None, pin: bool = True) -> torch.Tensor:
    size = lib().ckpt_file_size(_b(path))
    _check(int(size) if size < 0 else 0, "ckpt_file_size")
    if buf is None:
        buf = torch.empty(size, dtype=torch.uint8, pin_memory=pin)
    _check(lib().ckpt_file_read(_b(path), _host_u8(buf, "buf"), buf.numel()), "ckpt_file_read")
    return buf


def ckpt_file_latest(directory):
    """(step, path) of the newest valid step file, or None."""
    step = ctypes.c_int32(-1)
    out = ctypes.create_string_buffer(4096)
    rc = lib().ckpt_file_latest(_b(directory), ctypes.byref(step), out, 4096)
    if rc == ENOENT:
        return None
    _check(rc, "ckpt_file_latest")
    return step.value, os.fsdecode(out.value)


def ckpt_file_rotate(directory, keep: int) -> int:
    return _check(lib().ckpt_file_rotate(_b(directory), int(keep)), "ckpt_file_rotate")


def signals_install() -> None:
    _check(lib().rcs_signals_install(), "rcs_signals_install")


def signals_poll() -> int:
    return lib().rcs_signals_poll()


class CkptWriter:
    """The library's asynchronous step-file writer (rcs_ckpt_writer_*): it owns
    a device snapshot, two pinned host images, a copy stream and a worker
    thread that writes <dir>/step_NNNNNN.bin atomically and keeps the newest
    `keep`."""

    def __init__(self, directory, n: int, keep: int = 3):
        os.makedirs(directory, exist_ok=True)
        h = ctypes.c_void_p()
        _check(lib().rcs_ckpt_writer_create(_b(directory), int(n), int(keep), ctypes.byref(h)),
               "rcs_ckpt_writer_create")
        self._h, self.n = h, int(n)

    def submit(self, step: int, w, m, v, stream=None) -> None:
        """Snapshot of (w, m, v) on the stream, then copy and write in the
        background; waits only while the host image it reuses is still being
        written; raises first if an earlier write failed."""
        if self._h is None:
            raise ValueError("writer is closed")
        n = self.n
        ptrs = (_dev_f32(w, "w", n), _dev_f32(m, "m", n), _dev_f32(v, "v", n))
        _check(lib().rcs_ckpt_writer_submit(self._h, int(step), *ptrs, _stream(stream)),
               "rcs_ckpt_writer_submit")

    def wait(self) -> str:
        """Waits for the writes in flight; returns the newest path written
        since the last wait ("" if none) or raises a failure."""
        if self._h is None:
            return ""
        out = ctypes.create_string_buffer(4096)
        _check(lib().rcs_ckpt_writer_wait(self._h, out, 4096), "rcs_ckpt_writer_wait")
        return os.fsdecode(out.value)

    def close(self) -> None:
        if self._h is not None:
            h, self._h = self._h, None
            _check(lib().rcs_ckpt_writer_destroy(h), "rcs_ckpt_writer_destroy")

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class StepFileCheckpointer:
    """Step-file policy around a training loop: call after_step(t, w, m, v)
    after every completed update. It writes <dir>/step_NNNNNN.bin when t is a
    multiple of `every` (0 = never by cadence), when SIGUSR1 arrived (write and
    continue) or when SIGTERM arrived (write, then after_step returns True:
    the caller exits), keeps the newest `keep` files, and resume() loads the
    newest valid one.

    async_write=True hands each save to the library's CkptWriter (a device
    snapshot on the training stream, the copy on its own stream, the atomic
    write and rotation on its worker thread), so training continues during
    both the host-link copy and the disk write; a save waits only while the
    writer's host image it reuses is still being written (two saves back). A
    SIGTERM save and flush() wait for every write in flight; a failed write
    raises from a later save or from flush()."""

    def __init__(self, directory, n: int, every: int = 100, keep: int = 3,
                 install_signals: bool = True, stream=None, async_write: bool = False):
        self.dir, self.n, self.every, self.keep = directory, int(n), int(every), int(keep)
        os.makedirs(directory, exist_ok=True)
        self.stream = stream
        self.written: list[str] = []  # files saved (asynchronous ones once submitted)
        self.async_write = bool(async_write)
        self._buf: torch.Tensor | None = None  # pinned host image, made on first use
        self._writer = CkptWriter(directory, self.n, self.keep) if self.async_write else None
        if install_signals:
            signals_install()

    @property
    def buf(self) -> torch.Tensor:
        """Pinned host image of a step file (synchronous saves and resume; the
        asynchronous writer has its own)."""
        if self._buf is None:
            self._buf = torch.empty(ckpt_bytes(self.n), dtype=torch.uint8, pin_memory=True)
        return self._buf

    def flush(self) -> None:
        """Waits for the asynchronous writes in flight and raises a failure."""
        if self._writer is not None:
            self._writer.wait()

    def close(self) -> None:
        """flush(), then frees the asynchronous writer."""
        self.flush()
        if self._writer is not None:
            self._writer.close()
            self._writer = None
            self.async_write = False

    def save(self, t: int, w, m, v, wait: bool = False) -> None:
        if self._writer is None:
            ckpt_pack(t, w, m, v, self.buf, stream=self.stream)
            torch.cuda.synchronize()
            self.written.append(ckpt_file_write(self.dir, self.buf))
            ckpt_file_rotate(self.dir, self.keep)
            return
        self._writer.submit(t, w, m, v, stream=self.stream)
        self.written.append(os.path.join(os.fspath(self.dir), step_file_name(t)))
        if wait:
            self.flush()

    def after_step(self, t: int, w, m, v) -> bool:
        sig = signals_poll()
        exiting = bool(sig & SIG_WRITE_EXIT)
        if sig or (self.every > 0 and t % self.every == 0):
            self.save(t, w, m, v, wait=exiting)
        return exiting

    def resume(self, w, m, v) -> int:
        """Loads the newest valid step file into w, m, v; returns its step
        (0 when there is none: a fresh run). Continue with t = step + 1."""
        self.flush()
        found = ckpt_file_latest(self.dir)
        if found is None:
            return 0
        _, path = found
        ckpt_file_read(path, self.buf)
        step = ckpt_unpack(self.buf, w, m, v, stream=self.stream)
        torch.cuda.synchronize()
        return step


def profile_enable(on: bool, max_records: int = 4096, every: int = 1) -> None:
    """Per-kernel HIP events inside adamw_clip_step on one call in `every`."""
    _check(lib().rcs_profile_enable(1 if on else 0, max_records, every), "rcs_profile_enable")


def profile_read():
    """(norm ms total, update ms total, recorded steps); synchronizes events."""
    a, b, k = ctypes.c_double(), ctypes.c_double(), ctypes.c_int64()
    _check(lib().rcs_profile_read(ctypes.byref(a), ctypes.byref(b), ctypes.byref(k)),
           "rcs_profile_read")
    return a.value, b.value, k.value
