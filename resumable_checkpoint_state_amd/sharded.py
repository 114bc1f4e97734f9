"""Sharded checkpoint with a manifest (Phase 19 lesson 80, checkpoint-sharded-
resume: "Concept", the manifest schema, "Atomic write", and the three failure
modes the schema must guard against).

Each rank owns a contiguous slice [param_shard_offset, + param_shard_numel) of
the flat parameter vector and writes its slice of (w, m, v) as its own step
file (the same [int32 step][int32 n][w][m][v] layout, n = the slice's size)
through the library's atomic write; the manifest is written last, also
atomically, so a crash never leaves a manifest that points at partial shards.
On one GPU the ranks are simulated in one process, as the lesson's own test
does; each rank's pack is the library's ckpt_pack of its slice.

Loading refuses, loudly: a world size other than the expected one, a shard
count that differs from the world size, shards that do not tile [0, n), and a
shard whose bytes do not hash to the manifest's sha256 (partial or corrupted
write).

The file layer is host-side orchestration around the C ABI (sha256 from
hashlib); all device work is the library's pack/unpack.
"""
from __future__ import annotations

import ctypes
import dataclasses
import hashlib
import json
import os

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


def save_sharded(directory, step: int, w, m, v, world_size: int,
                 wall_clock_seconds: float = 0.0, stream=None) -> ShardManifest:
    """Writes rank{r}.bin for every simulated rank, then manifest.json."""
    os.makedirs(directory, exist_ok=True)
    n = w.numel()
    shards = []
    for r, (off, numel) in enumerate(shard_ranges(n, world_size)):
        buf = torch.empty(ckpt_bytes(numel), dtype=torch.uint8, pin_memory=True)
        ckpt_pack(step, w[off:off + numel], m[off:off + numel], v[off:off + numel], buf,
                  stream=stream)
        torch.cuda.synchronize()
        name = f"rank{r}.bin"
        _check(lib().ckpt_file_write_path(_b(os.path.join(directory, name)),
                                          _host_u8(buf, "buf"), buf.numel()),
               "ckpt_file_write_path")
        digest = hashlib.sha256(buf.numpy()).hexdigest()
        shards.append(ShardEntry(r, name, digest, off, numel))
        del buf
    man = ShardManifest(world_size, int(step), float(wall_clock_seconds), shards)
    _write_atomic(os.path.join(directory, MANIFEST), man.to_json().encode())
    return man


def verify_sharded(directory, expected_world_size: int, n: int):
    """Reads and checks the manifest and every shard; returns (manifest, list
    of host byte buffers in rank order). Host-only: no device is touched."""
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
    shards = sorted(man.shards, key=lambda s: s.rank)
    if [s.rank for s in shards] != list(range(man.world_size)):
        raise ShardError("shard ranks are not 0..world_size-1")
    off = 0
    for s in shards:
        if s.param_shard_offset != off or s.param_shard_numel <= 0:
            raise ShardError(f"rank {s.rank}: shards do not tile the parameter vector")
        off += s.param_shard_numel
    if off != n:
        raise ShardError(f"shards cover {off} parameters, expected {n}")
    bufs = []
    for s in shards:
        if os.path.basename(s.path) != s.path or s.path in ("", ".", ".."):
            raise ShardError(f"rank {s.rank}: shard path {s.path!r} is not a plain file name")
        fpath = os.path.join(directory, s.path)
        if not os.path.exists(fpath):
            raise ShardError(f"rank {s.rank}: missing shard file {s.path}")
        with open(fpath, "rb") as f:
            raw = f.read()
        if hashlib.sha256(raw).hexdigest() != s.sha256:
            raise ShardError(f"rank {s.rank}: sha256 mismatch (partial or corrupted write)")
        if len(raw) != ckpt_bytes(s.param_shard_numel):
            raise ShardError(f"rank {s.rank}: {len(raw)} bytes for {s.param_shard_numel} params")
        h_step = int.from_bytes(raw[0:4], "little", signed=True)
        h_n = int.from_bytes(raw[4:8], "little", signed=True)
        if h_step != man.step or h_n != s.param_shard_numel:
            raise ShardError(f"rank {s.rank}: header (step {h_step}, n {h_n}) disagrees with "
                             f"the manifest (step {man.step}, n {s.param_shard_numel})")
        bufs.append(raw)
    return man, bufs


def load_sharded(directory, expected_world_size: int, w, m, v, stream=None) -> int:
    """Verifies everything first, then unpacks each shard into its slice of
    w, m, v; returns the step (continue with t = step + 1)."""
    man, bufs = verify_sharded(directory, expected_world_size, w.numel())
    for s, raw in zip(sorted(man.shards, key=lambda e: e.rank), bufs):
        host = torch.empty(len(raw), dtype=torch.uint8, pin_memory=True)
        host.numpy()[:] = np.frombuffer(raw, dtype=np.uint8)
        a, k = s.param_shard_offset, s.param_shard_numel
        ckpt_unpack(host, w[a:a + k], m[a:a + k], v[a:a + k], stream=stream)
        torch.cuda.synchronize()
    return man.step
