#!/usr/bin/env python3
"""Throughput of the fused clip+AdamW step on one MI355X.

One step = the whole per-update hot path on one batch of synthetic gradients:
host scalars, grad_norm_partial, grad_norm_final and the fused AdamW update,
all through the C ABI (adamw_clip_step). Inputs are resident in HBM before the
timed region starts: four gradient buffers are generated up front and used in
rotation. Prints one JSON line.

Byte model (algorithmic, per parameter per step): norm pass reads g (4 B);
the update reads w, g, m, v (16 B) and writes w, m, v (12 B): 32 B in all,
28 B of it in the update kernel.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused clip+AdamW params/s and HBM GB/s (% of peak) at n=124.4M fp32"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, vendor figure
UPDATE_BYTES_PER_PARAM = 28
STEP_BYTES_PER_PARAM = 32
PMC_SUMMARY = os.path.join(ROOT, "profiles", "adamw_update_vec_andrea120m_pmc.md")
CONFIG_WORKLOADS = ("flat262k", "andrea12m", "andrea120m_stress", "flat2e9")
KERNEL_SRC = os.path.join(ROOT, "resumable_checkpoint_state_amd", "csrc", "rcs.hip")


def _log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


HOST_SIDE_MARK = b"// ---------------------------------------------------------------- host side"


def kernel_source_hash(text: bytes | None = None) -> str:
    """sha256[:16] of the device part of rcs.hip (everything before its host
    side: launch constants and kernels) with comments and whitespace runs
    removed, so host-only and comment-only edits keep the counters."""
    if text is None:
        with open(KERNEL_SRC, "rb") as f:
            text = f.read()
    cut = text.find(HOST_SIDE_MARK)
    code = text if cut < 0 else text[:cut]
    code = re.sub(rb"/\*.*?\*/", b" ", code, flags=re.S)  # the device part has no string literals
    code = re.sub(rb"//[^\n]*", b" ", code)
    code = re.sub(rb"\s+", b" ", code).strip()
    return hashlib.sha256(code).hexdigest()[:16]


def pmc_summary_for(workload: str, n: int) -> str:
    """The counter summary of the update kernel that runs at n for this workload."""
    return os.path.join(ROOT, "profiles", f"{update_kernel_name(n)}_{workload}_pmc.md")


def measured_traffic(path: str = PMC_SUMMARY):
    """HBM bytes per update launch from a committed rocprofv3 counter summary,
    or None when there is none or the kernel source changed since."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        text = f.read()
    h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not h or not t or h.group(1) != kernel_source_hash():
        return None
    return float(t.group(1))


def cpu_baseline(wl, budget_s: float):
    """The oracle, untuned, single-threaded on this host: full-size steps of
    the same workload until about budget_s seconds have passed."""
    import numpy as np

    import oracle
    import workloads

    n = wl.n
    w = workloads.init_params(wl).numpy()
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    g = workloads.grads(wl, 1).numpy()
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    cpu_model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    allowed = sorted(os.sched_getaffinity(0))
    os.sched_setaffinity(0, {allowed[-1]})  # one core for the single-threaded oracle
    try:
        steps, t0 = 0, time.perf_counter()
        while True:
            oracle.adamw_clip_step(w, g, m, v, steps + 1, wl.lr, wl.wd, wl.clip)
            steps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or steps >= 100:
                break
    finally:
        os.sched_setaffinity(0, set(allowed))
    return {"value": n * steps / el, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} full {wl.name} steps (n={n:,}) on one host thread pinned to "
                      f"core {allowed[-1]}, {el:.1f} s",
            "host_cpu": cpu_model, "host_cores_available": len(allowed),
            "GBps_32B_per_param": 32 * n * steps / el / 1e9}


def async_pack_overlap(rcs, step, stream, w, m, v, buf, n, k=60):
    """K update steps alone, then the same K steps with an asynchronous pack
    (device snapshot + copy-stream drain) issued before them; the pack's
    host-link time should hide behind the steps."""
    import torch

    snap = torch.empty(rcs.ckpt_snapshot_bytes(n) // 4, device=w.device)
    copy_stream = torch.cuda.Stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rcs.ckpt_pack_async(0, w, m, v, snap, buf, compute_stream=stream, copy_stream=copy_stream)
    rcs.ckpt_pack_wait(snap)  # first touch
    torch.cuda.synchronize()
    # the snapshot kernel alone: the compute stream's share of an async pack
    snaps = []
    for _ in range(3):
        e0.record(stream)
        rcs.ckpt_pack_async(0, w, m, v, snap, buf, compute_stream=stream,
                            copy_stream=copy_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        snaps.append(e0.elapsed_time(e1))
    snap_ms = sorted(snaps)[1]
    e0.record(stream)
    for _ in range(k):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    alone = e0.elapsed_time(e1)
    t0 = time.perf_counter()
    e0.record(stream)
    rcs.ckpt_pack_async(0, w, m, v, snap, buf, compute_stream=stream, copy_stream=copy_stream)
    for _ in range(k):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    both_wall = (time.perf_counter() - t0) * 1e3
    with_pack = e0.elapsed_time(e1)
    return {"async_pack_steps": k, "steps_ms_alone": alone,
            "steps_ms_with_async_pack": with_pack, "wall_ms_steps_and_pack": both_wall,
            "snapshot_ms": snap_ms, "snapshot_GBps_24B_per_param": 24 * n / snap_ms / 1e6}


def writer_cadence(rcs, step, stream, w, m, v, n, every=10, submits=4):
    """The library's asynchronous writer at a cadence far shorter than one
    disk write: `every` update steps between submits. Each submit's host
    blocking time: it waits only while the host image it reuses (two
    submits back) is still being written, so the first two return at once."""
    import shutil
    import tempfile

    import torch

    d = tempfile.mkdtemp(prefix="rcs_writer_", dir=os.environ.get("TMPDIR", "/tmp"))
    try:
        wr = rcs.CkptWriter(d, n, keep=2)
        blocks = []
        for k in range(submits):
            for _ in range(every):
                step()
            t0 = time.perf_counter()
            wr.submit(k + 1, w, m, v, stream=stream)
            blocks.append((time.perf_counter() - t0) * 1e3)
        t0 = time.perf_counter()
        wr.wait()
        drain = (time.perf_counter() - t0) * 1e3
        torch.cuda.synchronize()
        wr.close()
    finally:
        shutil.rmtree(d, ignore_errors=True)
    return {"writer_cadence_steps": every, "writer_submit_block_ms": blocks,
            "writer_drain_ms": drain}


def sharded_rate(rcs, w, m, v, world=8):
    """Save and load of a sharded checkpoint (world simulated ranks) through
    one ShardedCheckpointer: per-rank pack into its staging buffer, atomic
    shard writes with fsync, sha256, the manifest as the commit; load verifies
    every shard, then reads each again and unpacks it."""
    import shutil
    import tempfile

    from resumable_checkpoint_state_amd import sharded

    d = tempfile.mkdtemp(prefix="rcs_shards_", dir=os.environ.get("TMPDIR", "/tmp"))
    try:
        ck = sharded.ShardedCheckpointer(d, w.numel(), world)  # staging made here, once
        t0 = time.perf_counter()
        ck.save(1, w, m, v)
        t_save = time.perf_counter() - t0
        t0 = time.perf_counter()
        ck.save(2, w, m, v)  # replaces the first: commit, then the old shards go
        t_save2 = time.perf_counter() - t0
        t0 = time.perf_counter()
        ck.load(w, m, v)
        t_load = time.perf_counter() - t0
    finally:
        shutil.rmtree(d, ignore_errors=True)
    return {"sharded_world": world, "sharded_save_ms": t_save * 1e3,
            "sharded_second_save_ms": t_save2 * 1e3, "sharded_load_ms": t_load * 1e3}


def file_write_rate(rcs, buf):
    """Atomic write of one packed step file (tmp + fsync + rename) to TMPDIR."""
    import shutil
    import tempfile

    d = tempfile.mkdtemp(prefix="rcs_bench_", dir=os.environ.get("TMPDIR", "/tmp"))
    try:
        t0 = time.perf_counter()
        rcs.ckpt_file_write(d, buf)
        dt = time.perf_counter() - t0
    finally:
        shutil.rmtree(d, ignore_errors=True)
    return {"file_write_GBps_with_fsync": buf.numel() / dt / 1e9, "file_write_ms": dt * 1e3}


def copy_calibration(gib: float, reps: int) -> None:
    """A plain device copy of known size, for scaling rocprofv3 byte counters."""
    import torch

    nbytes = int(gib * (1 << 30))
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": nbytes, "bytes_written": nbytes,
                      "reps": reps}))


def torch_reference(torch, wl, w, grads, steps: int) -> dict:
    """PyTorch's own fused AdamW after its global-norm clip, on one float32
    parameter of the same size with the same gradients, timed the same way on
    the current stream: a speed reference on the same GPU, not a parity one
    (its clip adds 1e-6 to the norm and its AdamW orders the float32 work
    differently)."""
    p = torch.nn.Parameter(w.detach().clone())
    opt = torch.optim.AdamW([p], lr=wl.lr, betas=(0.9, 0.999), eps=1e-8,
                            weight_decay=wl.wd, fused=True)
    k = 0

    def step():
        nonlocal k
        p.grad = grads[k % len(grads)]
        k += 1
        torch.nn.utils.clip_grad_norm_([p], wl.clip, foreach=True)
        opt.step()

    for _ in range(5):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / steps * 1e3
    del opt, p
    torch.cuda.empty_cache()

    # PyTorch's own streaming kernels on float32[n] buffers, for the roofline's
    # context: read/written bytes over time, GB/s
    a, b = grads[0], grads[1]
    c, d = torch.empty_like(a), torch.empty_like(a)
    nb = 4 * a.numel()
    ops = {"copy_1r1w": (lambda: c.copy_(a), 2 * nb),
           "add_2r1w": (lambda: torch.add(a, b, out=c), 3 * nb),
           "addcmul_3r1w": (lambda: torch.addcmul(a, b, c, out=d), 4 * nb),
           "sum_1r": (lambda: a.sum(), nb)}
    streaming = {}
    for name, (fn, nbytes) in ops.items():
        for _ in range(3):
            fn()
        e0.record()
        for _ in range(20):
            fn()
        e1.record()
        torch.cuda.synchronize()
        streaming[name] = nbytes / (e0.elapsed_time(e1) / 20 / 1e3) / 1e9
    del c, d
    torch.cuda.empty_cache()
    return {"us_per_step": us, "params_per_s": w.numel() / us * 1e6, "steps": steps,
            "what": "torch.nn.utils.clip_grad_norm_(foreach=True) + "
                    "torch.optim.AdamW(fused=True), float32, same n and gradients",
            "streaming_GBps": streaming}


def measure_steps(torch, rcs, step, stream, steps: int) -> dict:
    """Times `steps` calls of step() on `stream` three ways: the timed region
    itself (events around all of them, nothing else instrumented), the same
    again with every step's kernel dispatches stamping HIP events (the norm
    kernels' and the update kernel's start and end, on the stream they run
    on: the per-kernel averages over all `steps` launches), and with an event
    between consecutive steps (median and p90 per step)."""
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = ev0.elapsed_time(ev1) / steps

    rcs.profile_enable(True, max(steps, 1), 1)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step_ev = ev0.elapsed_time(ev1) / steps
    norm_ms, upd_ms, rec = rcs.profile_read()
    rcs.profile_enable(False)

    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for k in range(steps):
        step()
        evs[k + 1].record(stream)
    torch.cuda.synchronize()
    per_step = sorted(evs[k].elapsed_time(evs[k + 1]) * 1e3 for k in range(steps))
    return {"ms_step": ms_step, "ms_step_kernel_events": ms_step_ev, "wall_s": wall,
            "median_us": per_step[len(per_step) // 2],
            "p90_us": per_step[min(len(per_step) - 1, (9 * len(per_step)) // 10)],
            "norm_us": norm_ms / rec * 1e3, "update_us": upd_ms / rec * 1e3, "recorded": rec}


def host_cost(torch, rcs, step, stream, w, g, m, v, wl, calls: int = 200) -> dict:
    """Host time per enqueued update where the step is launch-bound: through
    the Python binding (argument checks on the tensors, then the C call) and
    through the C ABI with the pointers already extracted (ctypes only); the
    library's own host work (validation, workspace lookup, two launches) is in
    both. Wall time of `calls` back-to-back calls after a synchronize."""
    L = rcs.lib()
    ptrs = (w.data_ptr(), g.data_ptr(), m.data_ptr(), v.data_ptr())
    n, raw = w.numel(), stream.cuda_stream
    out = {}
    for label, fn in (("binding", lambda t: rcs.adamw_clip_step(w, g, m, v, t, wl.lr, wl.wd,
                                                                 wl.clip, stream=stream)),
                      ("c_abi", lambda t: L.adamw_clip_step(*ptrs, n, t, wl.lr, wl.wd, wl.clip,
                                                            raw))):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(calls):
            fn(k + 1)
        out[label] = (time.perf_counter() - t0) / calls * 1e6
        torch.cuda.synchronize()
    return out


def update_kernel_name(n: int) -> str:
    # the arrays here are 16-byte aligned; up to 8,388,608 elements the library's
    # update kernel also does the final norm reduction (two launches per step)
    return "adamw_update_vec_fold" if 4 <= n <= 8_388_608 else "adamw_update_vec"


def config_leg(torch, rcs, workloads, name: str, steps: int, warmup: int,
               cpu_seconds: float | None) -> dict:
    """One more workload timed like the headline one (its own buffers, four
    gradient buffers in rotation, resident before timing), with its update
    kernel's roofline, then, unless cpu_seconds is None, the oracle on a
    bounded sample of it."""
    wl = workloads.WORKLOADS[name]
    n = wl.n
    dev = torch.device("cuda:0")
    _log(f"[bench] config {name} n={n:,}")
    w = workloads.init_params(wl, device=dev)
    m, v = workloads.zeros_like_state(n, device=dev)
    grads = [workloads.grads(wl, t, device=dev) for t in range(1, 5)]
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t = 0

    def step():
        nonlocal t
        t += 1
        rcs.adamw_clip_step(w, grads[(t - 1) % 4], m, v, t, wl.lr, wl.wd, wl.clip, stream=stream)

    for _ in range(warmup):
        step()
    meas = measure_steps(torch, rcs, step, stream, steps)
    host = host_cost(torch, rcs, step, stream, w, grads[0], m, v, wl) if n <= 1_000_000 else None
    achieved = UPDATE_BYTES_PER_PARAM * n / (meas["update_us"] / 1e6) / 1e9
    out = {"workload": name, "n_params": n, "steps": steps, "ms_per_step": meas["ms_step"],
           "params_per_s": n / (meas["ms_step"] / 1e3),
           "model_GBps": STEP_BYTES_PER_PARAM * n / (meas["ms_step"] / 1e3) / 1e9,
           "step_us_median": meas["median_us"], "step_us_p90": meas["p90_us"],
           "kernels_us": {"norm": meas["norm_us"], "adamw_update": meas["update_us"]},
           "roofline": {"bound": "hbm", "kernel": update_kernel_name(n), "achieved": achieved,
                        "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                        "traffic": measured_traffic(pmc_summary_for(name, n)),
                        "bytes_per_launch": UPDATE_BYTES_PER_PARAM * n},
           "description": wl.description}
    if host is not None:
        out["host_us_per_call"] = host
    # the streaming ceilings at this n on these buffers: at 2e9 the update's
    # pattern rate without cache help, at the small sizes the per-launch floor
    # of a kernel of the update's shape
    out["ceilings"] = ceilings(torch, n, (w, grads[0], m, v))
    out["update_vs_pattern_ceiling"] = (out["ceilings"]["pattern_4r3w_us"]
                                        / meas["update_us"])
    del w, m, v, grads
    torch.cuda.empty_cache()
    if cpu_seconds is None:
        out["cpu_baseline"] = None
        out["cpu_baseline_skipped"] = ("the oracle's state for 2e9 parameters (24 GB) plus its "
                                       "gradient does not fit a bounded host sample; its "
                                       "per-element rate is the ANDREA-120M figure")
    else:
        out["cpu_baseline"] = cpu_baseline(wl, cpu_seconds)
    return out


def _ceiling_lib():
    import ctypes

    path = os.path.join(ROOT, "resumable_checkpoint_state_amd", "libceilings.so")
    L = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.rcs_ceiling_blocks.argtypes = [i64]
    L.rcs_ceiling_blocks.restype = i64
    L.rcs_ceiling_time.argtypes = [ctypes.c_int, vp, vp, vp, vp, i64, vp, ctypes.c_int, vp,
                                   ctypes.POINTER(ctypes.c_double)]
    L.rcs_ceiling_time.restype = ctypes.c_int
    return L


def ceilings(torch, n: int, arrays=None, reps: int = 10) -> dict:
    """What the chip's HBM gives three streaming patterns over float32[n]:
    a read (the norm pass's shape), a copy and the update's 4-read/3-write
    pattern with one add per element (both in the update's shape), each the
    average of `reps` launches on the current stream, each stamped with its
    own start and stop events (as the library stamps the update's launches),
    so at small n they give the per-launch floor of each shape. `arrays` (w,
    g, m, v) are reused (and overwritten) when given."""
    import ctypes

    L = _ceiling_lib()
    n4 = n // 4
    made = arrays is None
    if made:
        arrays = [torch.ones(4 * n4, device="cuda") for _ in range(4)]
    p = [a.data_ptr() for a in arrays]
    out_buf = torch.empty(max(1, L.rcs_ceiling_blocks(n4)), device="cuda")
    st = torch.cuda.current_stream().cuda_stream

    def timed(kind):
        us = ctypes.c_double(0.0)
        rc = L.rcs_ceiling_time(kind, p[0], p[1], p[2], p[3], n4, out_buf.data_ptr(), reps, st,
                                ctypes.byref(us))
        assert rc == 0, f"rcs_ceiling_time({kind}) returned {rc}"
        return us.value / 1e6

    r, c, k = timed(0), timed(1), timed(2)
    if made:
        del arrays
        torch.cuda.empty_cache()
    return {"n": 4 * n4, "read_GBps": 16 * n4 / r / 1e9, "copy_GBps": 32 * n4 / c / 1e9,
            "pattern_4r3w_GBps": 112 * n4 / k / 1e9, "read_us": r * 1e6, "copy_us": c * 1e6,
            "pattern_4r3w_us": k * 1e6}


VIEW_OFFSETS = [(0, 0, 0, 0), (0, 1, 0, 0), (0, 0, 1, 0), (0, 0, 0, 1), (1, 0, 0, 0),
                (1, 2, 0, 0), (0, 1, 2, 3), (2, 0, 1, 3), (1, 1, 1, 1), (0, 0, 0, 4),
                (4, 0, 0, 0), (0, 0, 4, 4)]


def views_leg(torch, rcs, wl, steps: int, rounds: int = 3, only=None) -> dict:
    """The step on views of w, g, m, v at several element offsets (so at
    several 16- and 256-byte phases), with the buffers' physical placement
    held fixed: one set of padded buffers per round, every offset case timed
    on views into the same buffers, interleaved; mean us/step per case.
    only: one offset tuple to run alone, once (for counter runs)."""
    import ctypes

    n = wl.n
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if only is not None:
        bufs = [torch.zeros(n + 128, device="cuda") for _ in range(4)]
        bufs[0].normal_(0.0, 0.02)
        bufs[1].normal_(0.0, wl.grad_sigma)
        w, g, m, v = (b[o:o + n] for b, o in zip(bufs, only))
        e0.record(stream)
        for t in range(1, 1 + steps):
            rcs.adamw_clip_step(w, g, m, v, t, wl.lr, wl.wd, wl.clip, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return {"n": n, "offsets": list(only), "steps": steps,
                "us_per_step": e0.elapsed_time(e1) / steps * 1e3}
    times = {offs: [] for offs in VIEW_OFFSETS}
    # the bare 4-read/3-write pattern on the same buffers: all arrays on a line,
    # v 16 bytes past one with streaming accesses, and the same with
    # cache-retaining accesses on the lines two waves share
    lines = {"aligned": [], "v+16B_streaming": [], "v+16B_shared_lines_kept": []}
    L = _ceiling_lib()
    n4 = n // 4
    for _ in range(rounds):
        bufs = [torch.zeros(n + 128, device="cuda") for _ in range(4)]
        bufs[0].normal_(0.0, 0.02)
        bufs[1].normal_(0.0, wl.grad_sigma)
        for offs in VIEW_OFFSETS:
            w, g, m, v = (b[o:o + n] for b, o in zip(bufs, offs))
            for t in range(1, 4):
                rcs.adamw_clip_step(w, g, m, v, t, wl.lr, wl.wd, wl.clip, stream=stream)
            torch.cuda.synchronize()
            e0.record(stream)
            for t in range(4, 4 + steps):
                rcs.adamw_clip_step(w, g, m, v, t, wl.lr, wl.wd, wl.clip, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            times[offs].append(e0.elapsed_time(e1) / steps * 1e3)
        p = [b.data_ptr() for b in bufs]
        for label, kind, v_off in (("aligned", 2, 0), ("v+16B_streaming", 2, 16),
                                   ("v+16B_shared_lines_kept", 3, 16)):
            us = ctypes.c_double(0.0)
            rc = L.rcs_ceiling_time(kind, p[0], p[1], p[2], p[3] + v_off, n4, None, 10,
                                    stream.cuda_stream, ctypes.byref(us))
            assert rc == 0, f"rcs_ceiling_time({kind}) returned {rc}"
            lines[label].append(us.value)
        del bufs
        torch.cuda.empty_cache()
    base = sum(times[(0, 0, 0, 0)]) / rounds

    # the asynchronous pack's snapshot kernel at the same size: n % 4 == 0 with
    # everything aligned, n % 4 == 3 (the m and v parts off a 16-byte
    # boundary), and a snapshot buffer one float off (every source shifted)
    snaps = {}
    W, M, V = (torch.zeros(n + 4, device="cuda") for _ in range(3))
    S = torch.empty(3 * n + 8, device="cuda")
    host = torch.empty(rcs.ckpt_bytes(n), dtype=torch.uint8, pin_memory=True)
    copy_stream = torch.cuda.Stream()
    for label, nn, so in (("n%4=0", n, 0), ("n%4=3", n - 1, 0), ("snapshot+1", n, 1)):
        w, m, v, snap = W[:nn], M[:nn], V[:nn], S[so:so + 3 * nn]
        buf = host[:rcs.ckpt_bytes(nn)]
        ts = []
        for _ in range(4):
            e0.record(stream)
            rcs.ckpt_pack_async(0, w, m, v, snap, buf, compute_stream=stream,
                                copy_stream=copy_stream)
            e1.record(stream)
            rcs.ckpt_pack_wait(snap)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        snaps[label] = sorted(ts[1:])[1]  # median of the last three
    del W, M, V, S, host
    torch.cuda.empty_cache()
    return {"n": n, "steps": steps, "rounds": rounds, "snapshot_us": snaps,
            "pattern_4r3w_us": {k: sum(t) / rounds for k, t in lines.items()},
            "us_per_step": {",".join(map(str, o)): sum(t) / rounds for o, t in times.items()},
            "vs_aligned": {",".join(map(str, o)): sum(t) / rounds / base - 1
                           for o, t in times.items()},
            "what": "offsets of w, g, m, v in elements past 512-byte aligned buffers; "
                    "mean over rounds of fresh buffers, all cases on the same buffers per round"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="andrea120m")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-ckpt", action="store_true", help="skip the pack/unpack leg")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing the other workloads (small, ANDREA-12M, stress, 2e9)")
    ap.add_argument("--config-cpu-seconds", type=float, default=4.0,
                    help="oracle time budget per other workload")
    ap.add_argument("--no-torch-ref", action="store_true",
                    help="skip timing PyTorch's fused AdamW + clip on the same inputs")
    ap.add_argument("--views", action="store_true",
                    help="only time the step on views at several element offsets (fixed placement)")
    ap.add_argument("--view-offsets", default=None, metavar="W,G,M,V",
                    help="with --views: run only this offset case (elements), once")
    ap.add_argument("--calibrate-copy", type=float, default=0.0, metavar="GiB",
                    help="only run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0:
        print("bench.py needs --steps >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the update path runs per GPU and no "
              "multi-GPU leg (cross-GPU norm exchange, sharded state) is implemented; "
              "run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    import resumable_checkpoint_state_amd as rcs
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    if args.calibrate_copy > 0:
        copy_calibration(args.calibrate_copy, 10)
        return 0

    wl = workloads.WORKLOADS[args.workload]
    n = wl.n
    dev = torch.device("cuda:0")
    if args.views:
        rcs.lib()
        only = None
        if args.view_offsets is not None:
            only = tuple(int(x) for x in args.view_offsets.split(","))
            if len(only) != 4 or min(only) < 0 or max(only) > 127:
                print("--view-offsets takes four offsets 0..127", file=sys.stderr)
                return 2
        print(json.dumps({"views": views_leg(torch, rcs, wl, args.steps, only=only)}), flush=True)
        return 0
    rcs.lib()
    _log(f"[bench] workload {wl.name} n={n:,}: generating inputs on the device")
    w = workloads.init_params(wl, device=dev)
    m, v = workloads.zeros_like_state(n, device=dev)
    grads = [workloads.grads(wl, t, device=dev) for t in range(1, 5)]
    stream = torch.cuda.current_stream()
    rcs.init(0, stream)
    torch.cuda.synchronize()

    t = 0

    def step():
        nonlocal t
        t += 1
        rcs.adamw_clip_step(w, grads[(t - 1) % 4], m, v, t, wl.lr, wl.wd, wl.clip,
                            stream=stream)

    _log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K uninstrumented steps; then K more whose kernel dispatches
    # stamp HIP events (the kernel averages); then K with per-step events
    meas = measure_steps(torch, rcs, step, stream, args.steps)
    ms_step = meas["ms_step"]
    _log(f"[bench] timed {args.steps} steps: {ms_step * 1e3:.1f} us/step "
         f"(wall {meas['wall_s'] / args.steps * 1e6:.1f} us/step); kernel averages over "
         f"{meas['recorded']} instrumented steps")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    upd_s = meas["update_us"] / 1e6
    achieved = UPDATE_BYTES_PER_PARAM * n / upd_s / 1e9
    params_per_s = n / (ms_step / 1e3)
    model_gbps = STEP_BYTES_PER_PARAM * n / (ms_step / 1e3) / 1e9

    result = {
        "metric": METRIC,
        "value": params_per_s,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the pages time only whole training steps on other hardware: context
        "context": {"pages_training_steps_per_min": 6,
                    "what": "whole ANDREA-120M training step (forward, backward, update) "
                            "on one RTX 4090 in FP16, about 10 s per step; not this metric"},
        "dtype": "f32",
        "data": f"synthetic, seeded: {wl.description}; 4 gradient buffers used in "
                "rotation, inputs resident in HBM",
        "config": {"workload": wl.name, "n_params": n, "layout": wl.layout,
                   "lr": wl.lr, "wd": wl.wd, "clip": wl.clip, "grad_sigma": wl.grad_sigma},
        "model_GBps": model_gbps,
        "model_frac_of_hbm_peak": model_gbps / HBM_PEAK_GBPS,
        # norm: grad_norm_partial's start to the end of the last norm kernel
        # (grad_norm_final, or grad_norm_partial when the update folds it in)
        "kernels_us": {"norm": meas["norm_us"], "adamw_update": meas["update_us"]},
        "ms_per_step_with_kernel_events": meas["ms_step_kernel_events"],
        "step_us_median": meas["median_us"],
        "step_us_p90": meas["p90_us"],
        "roofline": {"bound": "hbm", "kernel": update_kernel_name(n), "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(pmc_summary_for(wl.name, n)),
                     "bytes_per_launch": UPDATE_BYTES_PER_PARAM * n},
    }

    # the clip on its own (norm kernels + in-place scale), 12 B/param
    reps = 10
    ev0.record(stream)
    for _ in range(reps):
        rcs.grad_clip_inplace(grads[0], wl.clip, stream=stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    clip_s = ev0.elapsed_time(ev1) / reps / 1e3
    result["grad_clip_inplace"] = {"us": clip_s * 1e6, "GBps_12B_per_param": 12 * n / clip_s / 1e9}

    # the accumulation buffer's reset after the step, 4 B/param written (on a
    # scratch buffer: the gradient buffers keep their contents)
    scratch = torch.empty(n, dtype=torch.float32, device=dev)
    rcs.grad_zero(scratch, stream=stream)
    ev0.record(stream)
    for _ in range(reps):
        rcs.grad_zero(scratch, stream=stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    zero_s = ev0.elapsed_time(ev1) / reps / 1e3
    result["grad_zero"] = {"us": zero_s * 1e6, "GBps_4B_per_param": 4 * n / zero_s / 1e9}
    del scratch

    # what the HBM gives the same streaming patterns at this size (fresh buffers)
    result["ceilings"] = ceilings(torch, n)
    result["update_vs_pattern_ceiling"] = result["ceilings"]["pattern_4r3w_us"] / meas["update_us"]

    if not args.no_torch_ref:
        ref = torch_reference(torch, wl, w, grads, min(args.steps, 50))
        ref["our_speedup"] = ref["us_per_step"] / (ms_step * 1e3)
        result["torch_reference"] = ref

    if not args.no_ckpt:
        nb = rcs.ckpt_bytes(n)
        buf = torch.empty(nb, dtype=torch.uint8, pin_memory=True)
        rcs.ckpt_pack(t, w, m, v, buf, stream=stream)  # first touch of the pinned pages
        torch.cuda.synchronize()
        reps = 3
        ev0.record(stream)
        for _ in range(reps):
            rcs.ckpt_pack(t, w, m, v, buf, stream=stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        pack_s = ev0.elapsed_time(ev1) / reps / 1e3
        ev0.record(stream)
        for _ in range(reps):
            rcs.ckpt_unpack(buf, w, m, v, stream=stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        unpack_s = ev0.elapsed_time(ev1) / reps / 1e3
        result["ckpt"] = {"bytes": nb, "pack_GBps_host_link": nb / pack_s / 1e9,
                          "unpack_GBps_host_link": nb / unpack_s / 1e9,
                          "pack_ms": pack_s * 1e3, "unpack_ms": unpack_s * 1e3}
        result["ckpt"].update(async_pack_overlap(rcs, step, stream, w, m, v, buf, n))
        for leg in (lambda: file_write_rate(rcs, buf), lambda: sharded_rate(rcs, w, m, v),
                    lambda: writer_cadence(rcs, step, stream, w, m, v, n)):
            try:  # a full or read-only TMPDIR must not cost the step measurement
                result["ckpt"].update(leg())
            except (OSError, RuntimeError) as e:
                result["ckpt"].setdefault("file_leg_errors", []).append(str(e))
        del buf

    if not args.no_cpu_baseline:
        _log(f"[bench] CPU baseline: the oracle for about {args.cpu_seconds:.0f} s")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)

    if not args.no_configs:
        # the other workloads, timed the same way after the headline one; the
        # headline's buffers are released first
        del w, m, v, grads
        torch.cuda.empty_cache()
        cpu_s = None if args.no_cpu_baseline else args.config_cpu_seconds
        result["configs"] = {
            name: config_leg(torch, rcs, workloads, name, args.steps, args.warmup,
                             None if name == "flat2e9" else cpu_s)
            for name in CONFIG_WORKLOADS if name != wl.name}

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
