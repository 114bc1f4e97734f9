"""Helpers shared by the tests: ulp distances and byte views."""
import numpy as np


def ordered(a: np.ndarray) -> np.ndarray:
    """float32 bits mapped to a monotone int64 line (sign-magnitude order):
    +-0 map to 0, adjacent floats (subnormals included) differ by 1."""
    i = np.ascontiguousarray(a, dtype=np.float32).view(np.int32).astype(np.int64)
    return np.where(i < 0, -(i & 0x7FFFFFFF), i)


def ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return np.abs(ordered(a) - ordered(b))


def max_ulp(a: np.ndarray, b: np.ndarray) -> int:
    if a.size == 0:
        return 0
    return int(ulp_diff(a, b).max())


def bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
