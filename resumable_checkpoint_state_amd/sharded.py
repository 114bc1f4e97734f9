"""Sharded checkpoint with a manifest (Phase 19 lesson 80, checkpoint-sharded-
resume: "Concept", the manifest schema, "Atomic write", and the three failure
modes the schema must guard against).

Each rank owns a contiguous slice [param_shard_offset, + param_shard_numel) of
the flat parameter vector and writes its slice of (w, m, v) as its own step
file (the same [int32 step][int32 n][w][m][v] layout, n = the slice's size)
through the library's atomic write (temporary file, fsync, rename, fsync of
the directory). Shard files are named for the step and for the save
(step_NNNNNN.rank{r}.{token}.bin), so a save never overwrites a file the
current manifest names; the new manifest is renamed into place only after
every shard is on disk, which is the single commit point, and only then are
the previous checkpoint's shard files removed. A crash anywhere during a save
leaves the previous checkpoint loadable.

One pinned staging buffer, sized to the largest shard, is made when a
ShardedCheckpointer is created and reused for every rank and every save and
load (the engine of the pages preallocates its buffers at start-up). On one
GPU the ranks are simulated in one process, as the lesson's own test does;
each rank's pack is the library's ckpt_pack of its slice.

Loading refuses, loudly and before any device memory is written: a world
size other than the expected one, a shard count that differs from the world
size, shards that do not tile [0, n), and a shard whose bytes do not hash to
the manifest's sha256 (partial or corrupted write).

The file layer is host-side orchestration around the C ABI (sha256 from
hashlib); all device work is the library's pack/unpack.
"""
from __future__ import annotations

import ctypes
import dataclasses
import hashlib
import json
import os
import re

import numpy as np
import torch

from . import _b, _check, _host_u8, ckpt_bytes, ckpt_pack, ckpt_unpack, lib

SCHEMA_VERSION = 1
MANIFEST = "manifest.json"


class ShardError(ValueError):
    """A sharded checkpoint that must not be loaded."""


@dataclasses.dataclass
class ShardEntry:
    rank: int
    path: str
    sha256: str
    param_shard_offset: int
    param_shard_numel: int


@dataclasses.dataclass
class ShardManifest:
    world_size: int
    step: int
    wall_clock_seconds: float
    shards: list[ShardEntry]
    schema_version: int = SCHEMA_VERSION

    def to_json(self) -> str:
        return json.dumps(dataclasses.asdict(self), indent=2)

    @staticmethod
    def from_json(text: str) -> "ShardManifest":
        try:  # bad JSON, missing keys, wrong types and non-numbers all refuse the load
            d = json.loads(text)
            shards = [ShardEntry(**s) for s in d["shards"]]
            return ShardManifest(world_size=int(d["world_size"]), step=int(d["step"]),
                                 wall_clock_seconds=float(d["wall_clock_seconds"]),
                                 shards=shards, schema_version=int(d["schema_version"]))
        except (KeyError, TypeError, ValueError) as e:
            raise ShardError(f"malformed manifest: {e}") from None


def shard_ranges(n: int, world_size: int) -> list[tuple[int, int]]:
    """Contiguous near-equal slices of [0, n); every boundary but the last is a
    multiple of 4 elements, so each slice starts 16-byte aligned."""
    if world_size < 1 or n < world_size:
        raise ValueError("need 1 <= world_size <= n")
    base = (n // world_size) // 4 * 4
    if base == 0:
        base = n // world_size
    out, off = [], 0
    for r in range(world_size):
        numel = base if r < world_size - 1 else n - off
        out.append((off, numel))
        off += numel
    return out


def _write_atomic(path: str, data: bytes) -> None:
    buf = ctypes.create_string_buffer(data, len(data))
    _check(lib().rcs_file_write_atomic(_b(path), buf, len(data)), "rcs_file_write_atomic")


def _read_manifest(directory, expected_world_size: int, n: int) -> ShardManifest:
    """The manifest with every check that needs no shard bytes."""
    path = os.path.join(directory, MANIFEST)
    if not os.path.exists(path):
        raise ShardError(f"no manifest in {directory} (checkpoint incomplete)")
    with open(path) as f:
        man = ShardManifest.from_json(f.read())
    if man.schema_version != SCHEMA_VERSION:
        raise ShardError(f"schema_version {man.schema_version}, expected {SCHEMA_VERSION}")
    if man.world_size != expected_world_size:
        raise ShardError(f"checkpoint was written by world_size={man.world_size}, "
                         f"loading with world_size={expected_world_size}")
    if len(man.shards) != man.world_size:
        raise ShardError(f"manifest lists {len(man.shards)} shards for "
                         f"world_size={man.world_size}")
    man.shards = sorted(man.shards, key=lambda s: s.rank)
    if [s.rank for s in man.shards] != list(range(man.world_size)):
        raise ShardError("shard ranks are not 0..world_size-1")
    off = 0
    for s in man.shards:
        if s.param_shard_offset != off or s.param_shard_numel <= 0:
            raise ShardError(f"rank {s.rank}: shards do not tile the parameter vector")
        off += s.param_shard_numel
        if os.path.basename(s.path) != s.path or s.path in ("", ".", ".."):
            raise ShardError(f"rank {s.rank}: shard path {s.path!r} is not a plain file name")
    if off != n:
        raise ShardError(f"shards cover {off} parameters, expected {n}")
    return man


def _read_shard(directory, man: ShardManifest, s: ShardEntry, out: np.ndarray) -> np.ndarray:
    """Reads shard s into out[:size] and checks its size, sha256 and header
    against the manifest; returns the filled view."""
    fpath = os.path.join(directory, s.path)
    if not os.path.exists(fpath):
        raise ShardError(f"rank {s.rank}: missing shard file {s.path}")
    size = os.path.getsize(fpath)
    want = ckpt_bytes(s.param_shard_numel)
    if size != want:
        raise ShardError(f"rank {s.rank}: {size} bytes for {s.param_shard_numel} params")
    if size > out.size:
        raise ShardError(f"rank {s.rank}: {size} bytes exceed the {out.size}-byte staging buffer")
    view = out[:size]
    with open(fpath, "rb", buffering=0) as f:
        got = f.readinto(memoryview(view))
    if got != size:
        raise ShardError(f"rank {s.rank}: short read of {s.path}")
    if hashlib.sha256(view).hexdigest() != s.sha256:
        raise ShardError(f"rank {s.rank}: sha256 mismatch (partial or corrupted write)")
    h_step = int.from_bytes(view[0:4].tobytes(), "little", signed=True)
    h_n = int.from_bytes(view[4:8].tobytes(), "little", signed=True)
    if h_step != man.step or h_n != s.param_shard_numel:
        raise ShardError(f"rank {s.rank}: header (step {h_step}, n {h_n}) disagrees with "
                         f"the manifest (step {man.step}, n {s.param_shard_numel})")
    return view


def verify_sharded(directory, expected_world_size: int, n: int,
                   staging: np.ndarray | None = None) -> ShardManifest:
    """Checks the manifest and every shard (size, sha256, header); returns the
    manifest. Host-only: no device is touched. staging: a uint8 buffer at
    least as large as the largest shard (one is made if absent)."""
    man = _read_manifest(directory, expected_world_size, n)
    if staging is None:
        staging = np.empty(max(ckpt_bytes(s.param_shard_numel) for s in man.shards), np.uint8)
    for s in man.shards:
        _read_shard(directory, man, s, staging)
    return man


class ShardedCheckpointer:
    """Sharded save and load of (w, m, v) over float32[n] for a fixed world
    size, through one pinned staging buffer made here and reused."""

    def __init__(self, directory, n: int, world_size: int, pin_memory: bool = True):
        """pin_memory=False makes a pageable staging buffer (host-only use,
        e.g. verifying files on a machine without a GPU)."""
        self.dir, self.n, self.world_size = str(directory), int(n), int(world_size)
        self.ranges = shard_ranges(self.n, self.world_size)
        self.pin_memory = bool(pin_memory)
        largest = max(ckpt_bytes(k) for _, k in self.ranges)
        self.staging = torch.empty(largest, dtype=torch.uint8, pin_memory=self.pin_memory)
        os.makedirs(self.dir, exist_ok=True)

    def save(self, step: int, w, m, v, wall_clock_seconds: float = 0.0,
             stream=None) -> ShardManifest:
        """Writes every rank's shard under a name of this save, then the
        manifest (the commit), then removes shard files the manifest does not
        name."""
        if w.numel() != self.n:
            raise ValueError(f"w has {w.numel()} elements, the checkpointer {self.n}")
        token = os.urandom(4).hex()
        shards = []
        for r, (off, numel) in enumerate(self.ranges):
            buf = self.staging[:ckpt_bytes(numel)]
            ckpt_pack(step, w[off:off + numel], m[off:off + numel], v[off:off + numel], buf,
                      stream=stream)
            torch.cuda.synchronize()
            name = f"step_{int(step):06d}.rank{r}.{token}.bin"
            _check(lib().ckpt_file_write_path(_b(os.path.join(self.dir, name)),
                                              _host_u8(buf, "buf"), buf.numel()),
                   "ckpt_file_write_path")
            shards.append(ShardEntry(r, name, hashlib.sha256(buf.numpy()).hexdigest(), off,
                                     numel))
        man = ShardManifest(self.world_size, int(step), float(wall_clock_seconds), shards)
        _write_atomic(os.path.join(self.dir, MANIFEST), man.to_json().encode())
        keep = {s.path for s in shards}
        for f in os.listdir(self.dir):
            if SHARD_FILE.fullmatch(f) and f not in keep:
                try:
                    os.remove(os.path.join(self.dir, f))
                except FileNotFoundError:
                    pass
        return man

    def load(self, w, m, v, stream=None) -> int:
        """Verifies every shard first (nothing is written to the device if any
        check fails), then reads each again, checks its hash again and unpacks
        it into its slice of w, m, v; returns the step (continue with
        t = step + 1)."""
        if w.numel() != self.n:
            raise ValueError(f"w has {w.numel()} elements, the checkpointer {self.n}")
        man = _read_manifest(self.dir, self.world_size, self.n)
        need = max(ckpt_bytes(s.param_shard_numel) for s in man.shards)
        if need > self.staging.numel():  # a checkpoint split differently from this one
            self.staging = torch.empty(need, dtype=torch.uint8, pin_memory=self.pin_memory)
        host = self.staging.numpy()
        for s in man.shards:
            _read_shard(self.dir, man, s, host)
        for s in man.shards:
            view = _read_shard(self.dir, man, s, host)
            a, k = s.param_shard_offset, s.param_shard_numel
            ckpt_unpack(self.staging[:view.size], w[a:a + k], m[a:a + k], v[a:a + k],
                        stream=stream)
            torch.cuda.synchronize()
        return man.step


# Shard files a save writes (and removes once a newer manifest is in place),
# with the atomic write's temporaries.
SHARD_FILE = re.compile(r"step_\d+\.rank\d+\.[0-9a-f]+\.bin(\.tmp)?")


def save_sharded(directory, step: int, w, m, v, world_size: int,
                 wall_clock_seconds: float = 0.0, stream=None) -> ShardManifest:
    """One save through a ShardedCheckpointer made for it."""
    return ShardedCheckpointer(directory, w.numel(), world_size).save(
        step, w, m, v, wall_clock_seconds, stream)


def load_sharded(directory, expected_world_size: int, w, m, v, stream=None) -> int:
    """One load through a ShardedCheckpointer made for it."""
    return ShardedCheckpointer(directory, w.numel(), expected_world_size).load(w, m, v, stream)
