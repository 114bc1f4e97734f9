"""Sharded checkpoint manifest: the three failure modes of the sharded-resume
lesson, checked on the host with shard files written by the oracle's pack
(no GPU needed), plus the GPU save/load round trip."""
import hashlib
import json
import os

import numpy as np
import pytest
import torch

import oracle
import resumable_checkpoint_state_amd as rcs
from resumable_checkpoint_state_amd import sharded


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(rcs.LIB_PATH):
        rcs.build()
    rcs.lib()


def _arrays(n, seed=0):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal(n).astype(np.float32) for _ in range(3)]


def _write_host_sharded(d, step, w, m, v, world):
    """A sharded checkpoint written with the oracle's pack and the manifest
    schema of the lesson, independently of the library's save path."""
    shards = []
    for r, (off, k) in enumerate(sharded.shard_ranges(w.size, world)):
        _, buf = oracle.ckpt_pack(step, w[off:off + k].copy(), m[off:off + k].copy(),
                                  v[off:off + k].copy())
        name = f"rank{r}.bin"
        open(os.path.join(d, name), "wb").write(buf.tobytes())
        shards.append({"rank": r, "path": name, "sha256": hashlib.sha256(buf).hexdigest(),
                       "param_shard_offset": off, "param_shard_numel": k})
    man = {"world_size": world, "step": step, "wall_clock_seconds": 12.5, "shards": shards,
           "schema_version": 1}
    open(os.path.join(d, "manifest.json"), "w").write(json.dumps(man))
    return man


def test_shard_ranges_tile_and_align():
    for n, world in [(262_144, 4), (1001, 4), (12_800_000, 8), (7, 7), (124_356_864, 8)]:
        rs = sharded.shard_ranges(n, world)
        assert rs[0][0] == 0 and sum(k for _, k in rs) == n
        for (a, k), (b, _) in zip(rs, rs[1:]):
            assert a + k == b
        if n >= 4 * world:
            assert all(a % 4 == 0 for a, _ in rs)


def test_verify_accepts_consistent_checkpoint(tmp_path):
    w, m, v = _arrays(1000)
    _write_host_sharded(tmp_path, 1234, w, m, v, 4)
    man = sharded.verify_sharded(tmp_path, 4, 1000)
    assert man.step == 1234 and man.world_size == 4 and len(man.shards) == 4
    bufs = [open(tmp_path / s.path, "rb").read() for s in man.shards]
    joined = np.concatenate([np.frombuffer(b[8:8 + 4 * s.param_shard_numel], np.float32)
                             for b, s in zip(bufs, man.shards)])
    assert (joined.view(np.uint32) == w.view(np.uint32)).all()


def test_world_size_change_is_refused(tmp_path):
    w, m, v = _arrays(1000)
    _write_host_sharded(tmp_path, 5, w, m, v, 4)
    with pytest.raises(sharded.ShardError, match="world_size"):
        sharded.verify_sharded(tmp_path, 8, 1000)


def test_shard_count_mismatch_is_refused(tmp_path):
    w, m, v = _arrays(1000)
    man = _write_host_sharded(tmp_path, 5, w, m, v, 4)
    man["shards"] = man["shards"][:3]
    open(tmp_path / "manifest.json", "w").write(json.dumps(man))
    with pytest.raises(sharded.ShardError, match="shards"):
        sharded.verify_sharded(tmp_path, 4, 1000)


@pytest.mark.parametrize("damage", ["truncate", "flip", "missing"])
def test_partial_or_corrupted_shard_is_refused(tmp_path, damage):
    w, m, v = _arrays(1000)
    _write_host_sharded(tmp_path, 5, w, m, v, 4)
    p = tmp_path / "rank2.bin"
    raw = bytearray(open(p, "rb").read())
    if damage == "truncate":
        open(p, "wb").write(raw[: len(raw) // 2])
    elif damage == "flip":
        raw[100] ^= 0x01
        open(p, "wb").write(raw)
    else:
        os.remove(p)
    with pytest.raises(sharded.ShardError, match="rank 2"):
        sharded.verify_sharded(tmp_path, 4, 1000)


def test_missing_manifest_means_incomplete(tmp_path):
    w, m, v = _arrays(100)
    _write_host_sharded(tmp_path, 5, w, m, v, 2)
    os.remove(tmp_path / "manifest.json")
    with pytest.raises(sharded.ShardError, match="incomplete"):
        sharded.verify_sharded(tmp_path, 2, 100)


def test_header_step_disagreeing_with_manifest_is_refused(tmp_path):
    w, m, v = _arrays(100)
    man = _write_host_sharded(tmp_path, 5, w, m, v, 2)
    man["step"] = 6
    open(tmp_path / "manifest.json", "w").write(json.dumps(man))
    with pytest.raises(sharded.ShardError, match="header"):
        sharded.verify_sharded(tmp_path, 2, 100)


@pytest.mark.parametrize("damage", ["truncated_json", "missing_key", "step_not_a_number",
                                    "shards_not_a_list", "extra_shard_field"])
def test_malformed_manifest_is_refused(tmp_path, damage):
    w, m, v = _arrays(100)
    man = _write_host_sharded(tmp_path, 5, w, m, v, 2)
    text = json.dumps(man)
    if damage == "truncated_json":
        text = text[: len(text) // 2]
    elif damage == "missing_key":
        del man["world_size"]
        text = json.dumps(man)
    elif damage == "step_not_a_number":
        man["step"] = "five"
        text = json.dumps(man)
    elif damage == "shards_not_a_list":
        man["shards"] = 7
        text = json.dumps(man)
    else:
        man["shards"][0]["owner"] = "someone"
        text = json.dumps(man)
    open(tmp_path / "manifest.json", "w").write(text)
    with pytest.raises(sharded.ShardError, match="malformed"):
        sharded.verify_sharded(tmp_path, 2, 100)


@pytest.mark.gpu
@pytest.mark.parametrize("world", [1, 3, 4, 8])
def test_gpu_save_load_round_trip_matches_oracle_shards(tmp_path, world):
    assert torch.cuda.is_available()
    n = 262_147
    w, m, v = _arrays(n, seed=world)
    dw, dm, dv = (torch.from_numpy(a).cuda() for a in (w, m, v))
    man = sharded.save_sharded(tmp_path, 80, dw, dm, dv, world, wall_clock_seconds=3.0)
    assert sorted(os.listdir(tmp_path)) == sorted(["manifest.json"] +
                                                  [s.path for s in man.shards])
    assert all(s.path.startswith(f"step_000080.rank{s.rank}.") for s in man.shards)
    for s in man.shards:  # every shard file is the oracle's pack of that slice
        a, k = s.param_shard_offset, s.param_shard_numel
        _, ob = oracle.ckpt_pack(80, w[a:a + k].copy(), m[a:a + k].copy(), v[a:a + k].copy())
        assert open(tmp_path / s.path, "rb").read() == ob.tobytes()
    out = [torch.full((n,), float("nan"), device="cuda") for _ in range(3)]
    assert sharded.load_sharded(tmp_path, world, *out) == 80
    for a, b in zip((dw, dm, dv), out):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    with pytest.raises(sharded.ShardError):
        sharded.load_sharded(tmp_path, world + 1, *out)


def _fake_ckpt(monkeypatch, fail_after_rank=None):
    """Routes the checkpointer's device pack through the oracle's pack of host
    arrays (no GPU), and can make the shard write fail after a given rank,
    as a crash in the middle of a save would."""
    def pack(step, w, m, v, buf, stream=None):
        _, ob = oracle.ckpt_pack(step, w.numpy().copy(), m.numpy().copy(), v.numpy().copy())
        buf.numpy()[:] = ob
        return buf

    monkeypatch.setattr(sharded, "ckpt_pack", pack)
    monkeypatch.setattr(sharded.torch.cuda, "synchronize", lambda *a, **k: None)
    real = rcs.lib().ckpt_file_write_path
    calls = {"n": 0}

    class Lib:
        def __getattr__(self, name):
            return getattr(rcs.lib(), name)

        def ckpt_file_write_path(self, path, buf, nbytes):
            if fail_after_rank is not None and calls["n"] > fail_after_rank:
                raise KeyboardInterrupt("simulated crash")
            calls["n"] += 1
            return real(path, buf, nbytes)

    monkeypatch.setattr(sharded, "lib", lambda: Lib())


def test_crash_during_a_save_keeps_the_previous_checkpoint(tmp_path, monkeypatch):
    """Save at step 80, then a save at step 160 that dies after rewriting
    rank 0 (and again after rank 2): the step-80 manifest and shards are
    untouched, verify and the shard bytes still give step 80."""
    n, world = 4000, 4
    w, m, v = (torch.from_numpy(a) for a in _arrays(n, seed=5))
    _fake_ckpt(monkeypatch)
    ck = sharded.ShardedCheckpointer(tmp_path, n, world, pin_memory=False)
    man80 = ck.save(80, w, m, v)
    before = {f: open(tmp_path / f, "rb").read() for f in os.listdir(tmp_path)}
    for fail_after in (0, 2):
        _fake_ckpt(monkeypatch, fail_after_rank=fail_after)
        ck = sharded.ShardedCheckpointer(tmp_path, n, world, pin_memory=False)
        with pytest.raises(KeyboardInterrupt):
            ck.save(160, w * 2, m * 2, v * 2)
        man = sharded.verify_sharded(tmp_path, world, n)
        assert man.step == 80 and [s.path for s in man.shards] == [s.path for s in man80.shards]
        for f, data in before.items():
            assert open(tmp_path / f, "rb").read() == data
    # a completed save then replaces it and removes the step-80 shards
    _fake_ckpt(monkeypatch)
    man160 = sharded.ShardedCheckpointer(tmp_path, n, world, pin_memory=False).save(
        160, w * 2, m * 2, v * 2)
    assert sharded.verify_sharded(tmp_path, world, n).step == 160
    left = sorted(os.listdir(tmp_path))
    assert left == sorted(["manifest.json"] + [s.path for s in man160.shards])


def test_checkpointer_reuses_one_staging_buffer(tmp_path, monkeypatch):
    """Every rank of every save goes through the buffer made at construction,
    sized to the largest shard."""
    n, world = 4003, 4
    w, m, v = (torch.from_numpy(a) for a in _arrays(n, seed=6))
    _fake_ckpt(monkeypatch)
    ck = sharded.ShardedCheckpointer(tmp_path, n, world, pin_memory=False)
    staging = ck.staging
    assert staging.numel() == max(rcs.ckpt_bytes(k) for _, k in sharded.shard_ranges(n, world))
    for step in (1, 2, 3):
        ck.save(step, w, m, v)
        assert ck.staging is staging
    assert sharded.verify_sharded(tmp_path, world, n).step == 3
