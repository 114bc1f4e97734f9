"""ctypes binding of the plain C oracle (oracle/oracle.c).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The product library
never imports it and shares no code with it.

Every function takes and returns numpy arrays on the host. The arithmetic is
all in oracle.c; this file only marshals arguments.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, SKIPPED, EINVAL, ESIZE, EHEADER = 0, 1, -1, -2, -3

_CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra"]


def build() -> str:
    """Compile oracle.c into liboracle.so with gcc (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    """The oracle library. RCS_ORACLE_LIB, when set, names another build of
    oracle.c to load instead: the mutation test plants one mistake in a copy of
    the source and checks that the pins catch it."""
    global _lib
    if _lib is None:
        path = os.environ.get("RCS_ORACLE_LIB") or _LIB
        if path == _LIB and not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(path)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        L.oracle_sumsq_accum.argtypes = [f64p, f32p, i64]
        L.oracle_sumsq_accum.restype = None
        L.oracle_sumsq_finish.argtypes = [f64p]
        L.oracle_sumsq_finish.restype = ctypes.c_double
        L.oracle_grad_norm.argtypes = [f32p, i64]
        L.oracle_grad_norm.restype = ctypes.c_double
        L.oracle_clip_scale.argtypes = [ctypes.c_double, ctypes.c_float]
        L.oracle_clip_scale.restype = ctypes.c_float
        L.oracle_scalars.argtypes = [i32, ctypes.c_float, ctypes.c_float, f32p, f32p, f32p]
        L.oracle_scalars.restype = None
        L.oracle_adamw_elems.argtypes = [f32p, f32p, f32p, f32p, i64, ctypes.c_float,
                                         ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                         ctypes.c_float]
        L.oracle_adamw_elems.restype = None
        L.oracle_adamw_clip_step.argtypes = [f32p, f32p, f32p, f32p, i64, i32, ctypes.c_float,
                                             ctypes.c_float, ctypes.c_float, f64p]
        L.oracle_adamw_clip_step.restype = ctypes.c_int
        L.oracle_adamw_clip_step_f64.argtypes = [f64p, f64p, f64p, f64p, i64, i32,
                                                 ctypes.c_double, ctypes.c_double,
                                                 ctypes.c_double, f64p]
        L.oracle_adamw_clip_step_f64.restype = ctypes.c_int
        L.oracle_ckpt_bytes.argtypes = [i64]
        L.oracle_ckpt_bytes.restype = i64
        L.oracle_ckpt_pack.argtypes = [i32, i64, f32p, f32p, f32p, u8p, i64]
        L.oracle_ckpt_pack.restype = ctypes.c_int
        L.oracle_ckpt_header.argtypes = [u8p, i64, ctypes.POINTER(i32), ctypes.POINTER(i32)]
        L.oracle_ckpt_header.restype = ctypes.c_int
        L.oracle_ckpt_unpack.argtypes = [u8p, i64, i64, ctypes.POINTER(i32), f32p, f32p, f32p]
        L.oracle_ckpt_unpack.restype = ctypes.c_int
        L.oracle_clip_grads.argtypes = [f32p, i64, ctypes.c_float, f64p]
        L.oracle_clip_grads.restype = ctypes.c_int
        L.oracle_scale_grads.argtypes = [f32p, i64, ctypes.c_float]
        L.oracle_scale_grads.restype = None
        L.oracle_subnormals_kept.argtypes = []
        L.oracle_subnormals_kept.restype = ctypes.c_int
        _lib = L
    return _lib


def _f32(a: np.ndarray, writable: bool = False):
    if a.dtype != np.float32 or not a.flags.c_contiguous:
        raise TypeError("expected a C-contiguous float32 array")
    if writable and not a.flags.writeable:
        raise TypeError("array must be writable")
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _u8(a: np.ndarray):
    if a.dtype != np.uint8 or not a.flags.c_contiguous:
        raise TypeError("expected a C-contiguous uint8 array")
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


class NormAccumulator:
    """Index-order compensated float64 sum of squares fed chunk by chunk."""

    def __init__(self):
        self._st = (ctypes.c_double * 2)(0.0, 0.0)

    def add(self, g: np.ndarray) -> None:
        lib().oracle_sumsq_accum(self._st, _f32(g), g.size)

    def sumsq(self) -> float:
        return lib().oracle_sumsq_finish(self._st)

    def norm(self) -> float:
        return float(np.sqrt(np.float64(self.sumsq())))


def grad_norm(g: np.ndarray) -> float:
    return lib().oracle_grad_norm(_f32(g), g.size)


def sumsq(g: np.ndarray) -> float:
    acc = NormAccumulator()
    acc.add(g)
    return acc.sumsq()


def clip_scale(norm: float, clip: float) -> np.float32:
    return np.float32(lib().oracle_clip_scale(norm, clip))


def scalars(t: int, lr: float, wd: float):
    """(bc1, bc2, decay) as float32 values."""
    b1, b2, d = ctypes.c_float(), ctypes.c_float(), ctypes.c_float()
    lib().oracle_scalars(t, lr, wd, ctypes.byref(b1), ctypes.byref(b2), ctypes.byref(d))
    return np.float32(b1.value), np.float32(b2.value), np.float32(d.value)


def adamw_elems(w, g, m, v, s, bc1, bc2, decay, lr) -> None:
    """In-place per-element update of w, m, v for a given clip factor s."""
    n = w.size
    assert g.size == n and m.size == n and v.size == n
    lib().oracle_adamw_elems(_f32(w, True), _f32(g), _f32(m, True), _f32(v, True), n,
                             s, bc1, bc2, decay, lr)


def adamw_clip_step(w, g, m, v, t: int, lr: float, wd: float, clip: float):
    """In-place full update. Returns (status, pre-clip norm)."""
    n = w.size
    assert g.size == n and m.size == n and v.size == n
    norm = ctypes.c_double(0.0)
    rc = lib().oracle_adamw_clip_step(_f32(w, True), _f32(g), _f32(m, True), _f32(v, True), n,
                                      t, lr, wd, clip, ctypes.byref(norm))
    return rc, norm.value


def clip_grads(g: np.ndarray, clip: float):
    """In place global clip; returns (status, pre-clip norm)."""
    norm = ctypes.c_double(0.0)
    rc = lib().oracle_clip_grads(_f32(g, True), g.size, clip, ctypes.byref(norm))
    return rc, norm.value


def scale_grads(g: np.ndarray, scale: float) -> None:
    """In place: g *= scale in float32 (micro-batch averaging)."""
    lib().oracle_scale_grads(_f32(g, True), g.size, scale)


def adamw_clip_step_accum(w, g_sum, m, v, t: int, lr: float, wd: float, clip: float,
                          grad_scale: float):
    """The pages' order: average the accumulated gradient (g *= grad_scale,
    float32), then the clipped update. g_sum is left untouched."""
    g = g_sum.copy()
    scale_grads(g, grad_scale)
    return adamw_clip_step(w, g, m, v, t, lr, wd, clip)


def _f64(a: np.ndarray, writable: bool = False):
    if a.dtype != np.float64 or not a.flags.c_contiguous:
        raise TypeError("expected a C-contiguous float64 array")
    if writable and not a.flags.writeable:
        raise TypeError("array must be writable")
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def adamw_clip_step_f64(w, g, m, v, t: int, lr: float, wd: float, clip: float):
    """The clipped AdamW definition in float64 over float64 arrays, in place.
    Returns (status, pre-clip norm)."""
    n = w.size
    assert g.size == n and m.size == n and v.size == n
    norm = ctypes.c_double(0.0)
    rc = lib().oracle_adamw_clip_step_f64(_f64(w, True), _f64(g), _f64(m, True), _f64(v, True),
                                          n, t, lr, wd, clip, ctypes.byref(norm))
    return rc, norm.value


def ckpt_bytes(n: int) -> int:
    return lib().oracle_ckpt_bytes(n)


def ckpt_pack(step: int, w, m, v, buf: np.ndarray | None = None):
    """Returns (status, buffer)."""
    n = w.size
    nb = ckpt_bytes(n)
    if buf is None:
        buf = np.zeros(max(nb, 0), dtype=np.uint8)
    rc = lib().oracle_ckpt_pack(step, n, _f32(w), _f32(m), _f32(v), _u8(buf), buf.size)
    return rc, buf


def ckpt_header(buf: np.ndarray):
    step, n = ctypes.c_int32(), ctypes.c_int32()
    rc = lib().oracle_ckpt_header(_u8(buf), buf.size, ctypes.byref(step), ctypes.byref(n))
    return rc, step.value, n.value


def ckpt_unpack(buf: np.ndarray, w, m, v):
    """Returns (status, step). The header's n must equal w.size; outputs are
    written only when status is OK."""
    n_expected = w.size
    if m.size != n_expected or v.size != n_expected or n_expected <= 0:
        raise ValueError("w, m, v must have the same positive size")
    step = ctypes.c_int32(-1)
    rc = lib().oracle_ckpt_unpack(_u8(buf), buf.size, n_expected, ctypes.byref(step),
                                  _f32(w, True), _f32(m, True), _f32(v, True))
    return rc, step.value


def subnormals_kept() -> bool:
    return bool(lib().oracle_subnormals_kept())
