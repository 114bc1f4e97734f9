"""GPU tests of the rows built on top of the hot path: micro-batch
accumulation folded into the kernels, the asynchronous snapshot pack, the
library's asynchronous step-file writer, and signal-driven step files with
resume."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
import resumable_checkpoint_state_amd as rcs
import workloads
from util import bits, max_ulp

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rcs.lib()
    torch.cuda.set_device(0)
    return torch.device("cuda:0")


def _host(t):
    return t.detach().cpu().numpy()


@pytest.mark.parametrize("n_micro,n", [(1, 1_000_003), (3, 1_000_003), (4, 1_000_003),
                                         (4, 124_356_864)])
def test_accumulated_microbatch_step_parity(dev, n_micro, n):
    wl = workloads.WORKLOADS["andrea12m"]
    w = workloads.init_params(wl, device=dev, n=n)
    m, v = workloads.zeros_like_state(n, device=dev)
    ow, om, ov = _host(w).copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    scale = float(np.float32(1.0) / np.float32(n_micro))
    for t in (1, 2, 3):
        g_sum = torch.zeros(n, device=dev)
        for k in range(n_micro):  # backward passes add into one buffer
            g_sum.add_(workloads.custom(200 + 10 * t + k, n, 0.05, device=dev))
        rcs.adamw_clip_step_accum(w, g_sum, m, v, t, wl.lr, wl.wd, wl.clip, scale)
        gn = float(rcs.last_grad_norm().cpu())
        rc, on = oracle.adamw_clip_step_accum(ow, _host(g_sum), om, ov, t, wl.lr, wl.wd, wl.clip,
                                              scale)
        assert rc == oracle.OK and on > wl.clip
        assert abs(gn - on) <= 1e-12 * on
        for name, a, b in (("w", w, ow), ("m", m, om), ("v", v, ov)):
            assert max_ulp(_host(a), b) <= 2, (n_micro, t, name)


@pytest.mark.parametrize("n,offset", [(1, 0), (3, 0), (5, 0), (4099, 0), (1_000_003, 0),
                                      (100_001, 1), (67, 1), (66, 1), (6, 1), (100_003, 17),
                                      (12_800_003, 2)])
def test_grad_zero_clears_exactly_the_view(dev, n, offset):
    """grad_zero writes +0.0 to every element of the view (vector kernel with
    heads of 1-63 elements and ragged tails, the 16-byte fallback and the
    scalar kernel) and nothing before or after it."""
    base = workloads.custom(950, n + offset + 5, 1.0, device=dev)
    before = _host(base).copy()
    rcs.grad_zero(base[offset:offset + n])
    torch.cuda.synchronize()
    after = _host(base)
    assert (bits(after[offset:offset + n]) == 0).all()
    assert (bits(after[:offset]) == bits(before[:offset])).all()
    assert (bits(after[offset + n:]) == bits(before[offset + n:])).all()


def test_accumulation_loop_reuses_one_buffer_with_grad_zero(dev):
    """The backprop lesson's loop on one gradient buffer: micro-batches add
    into it, the accumulated step reads it, grad_zero clears it for the next
    step. Three steps of three micro-batches against the oracle fed the same
    float32 sums."""
    n, n_micro = 1_000_003, 3
    wl = workloads.WORKLOADS["andrea12m"]
    w = workloads.init_params(wl, device=dev, n=n)
    m, v = workloads.zeros_like_state(n, device=dev)
    ow, om, ov = _host(w).copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    scale = float(np.float32(1.0) / np.float32(n_micro))
    g_sum = workloads.custom(299, n, 1.0, device=dev)  # stale contents from "before"
    rcs.grad_zero(g_sum)
    for t in (1, 2, 3):
        og = np.zeros(n, np.float32)
        for k in range(n_micro):
            mb = workloads.custom(300 + 10 * t + k, n, 0.05, device=dev)
            g_sum.add_(mb)
            og += _host(mb)
        rcs.adamw_clip_step_accum(w, g_sum, m, v, t, wl.lr, wl.wd, wl.clip, scale)
        rcs.grad_zero(g_sum)
        rc, on = oracle.adamw_clip_step_accum(ow, og, om, ov, t, wl.lr, wl.wd, wl.clip, scale)
        assert rc == oracle.OK
        for name, a, b in (("w", w, ow), ("m", m, om), ("v", v, ov)):
            assert max_ulp(_host(a), b) <= 2, (t, name)
        assert not bool(g_sum.any())


def test_accum_with_unit_scale_equals_plain_step(dev):
    n = 100_000
    wl = workloads.WORKLOADS["flat262k"]
    g = workloads.grads(wl, 1, device=dev, n=n).mul_(40)
    a = [workloads.init_params(wl, device=dev, n=n), *workloads.zeros_like_state(n, device=dev)]
    b = [x.clone() for x in a]
    rcs.adamw_clip_step(a[0], g, a[1], a[2], 1, wl.lr, wl.wd, wl.clip)
    rcs.adamw_clip_step_accum(b[0], g, b[1], b[2], 1, wl.lr, wl.wd, wl.clip, 1.0)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))


@pytest.mark.parametrize("n", [262_147, 12_800_000])
def test_async_pack_equals_synchronous_pack_while_training_continues(dev, n):
    """Snapshot at step k, keep updating on the compute stream while the copy
    stream drains; the bytes are the state at k. A second async pack out of
    the same snapshot buffer two steps later is ordered after the first copy."""
    wl = workloads.WORKLOADS["flat262k"]
    k = 5
    w = workloads.init_params(wl, device=dev, n=n)
    m, v = workloads.zeros_like_state(n, device=dev)
    ref = [w.clone(), m.clone(), v.clone()]
    g = torch.empty(n, device=dev)
    nb = rcs.ckpt_bytes(n)
    ref_bufs = {}
    for t in range(1, k + 3):  # reference: synchronous packs at k and k + 2
        workloads.grads(wl, t, device=dev, n=n, out=g)
        rcs.adamw_clip_step(ref[0], g, ref[1], ref[2], t, wl.lr, wl.wd, wl.clip)
        if t in (k, k + 2):
            ref_bufs[t] = torch.empty(nb, dtype=torch.uint8, pin_memory=True)
            rcs.ckpt_pack(t, *ref, ref_bufs[t])
    torch.cuda.synchronize()
    snap = torch.empty(rcs.ckpt_snapshot_bytes(n) // 4, device=dev)
    copy_stream = torch.cuda.Stream()
    bufs = {t: torch.empty(nb, dtype=torch.uint8, pin_memory=True) for t in (k, k + 2)}
    compute = torch.cuda.current_stream()
    for t in range(1, k + 12):
        workloads.grads(wl, t, device=dev, n=n, out=g)
        rcs.adamw_clip_step(w, g, m, v, t, wl.lr, wl.wd, wl.clip)
        if t in (k, k + 2):
            rcs.ckpt_pack_async(t, w, m, v, snap, bufs[t], compute_stream=compute,
                                copy_stream=copy_stream)
    rcs.ckpt_pack_wait(snap)
    torch.cuda.synchronize()
    for t in (k, k + 2):
        assert torch.equal(bufs[t], ref_bufs[t]), f"async pack at step {t} differs"
    # and the layout is the oracle's: repacking the arrays read out of it gives the same bytes
    _, ob = oracle.ckpt_pack(k, *[a.numpy() for a in _unpacked(bufs[k], n)])
    assert ob.tobytes() == bufs[k].numpy().tobytes()


# (n, offsets of w, m, v and the snapshot in elements past a 512-byte boundary):
# the snapshot's m and v parts start off a 16-byte boundary whenever n % 4 != 0,
# and views put the sources at other phases still; n < 4 takes the scalar copy.
SNAPSHOT_CASES = [(1, (0, 0, 0, 0)), (3, (1, 2, 3, 1)), (4, (0, 0, 0, 3)), (5, (0, 0, 0, 0)),
                  (7, (3, 2, 1, 0)), (262_147, (0, 0, 0, 0)), (262_146, (1, 1, 1, 1)),
                  (1_000_001, (2, 3, 0, 1)), (1_000_000, (0, 1, 2, 3))]


@pytest.mark.parametrize("n,offs", SNAPSHOT_CASES)
def test_async_pack_any_n_and_phase(dev, n, offs):
    """The snapshot kernel's 16-byte path at every 4-byte phase of source and
    destination: the async pack equals the synchronous pack of the same state,
    and the elements around the snapshot are not written."""
    W, M, V = (torch.zeros(n + 4, device=dev) for _ in range(3))
    S = torch.full((3 * n + 8,), 7.0, device=dev)
    w, m, v = (X[o:o + n] for X, o in zip((W, M, V), offs))
    snap = S[offs[3]:offs[3] + 3 * n]
    for x, seed in ((w, 1200), (m, 1201), (v, 1202)):
        x.copy_(workloads.custom(seed, n, 1.0, device=dev))
    nb = rcs.ckpt_bytes(n)
    ref, buf = (torch.empty(nb, dtype=torch.uint8, pin_memory=True) for _ in range(2))
    rcs.ckpt_pack(9, w, m, v, ref)
    copy_stream = torch.cuda.Stream()
    rcs.ckpt_pack_async(9, w, m, v, snap, buf, compute_stream=torch.cuda.current_stream(),
                        copy_stream=copy_stream)
    rcs.ckpt_pack_wait(snap)
    torch.cuda.synchronize()
    assert torch.equal(buf, ref), (n, offs)
    assert (S[:offs[3]] == 7.0).all() and (S[offs[3] + 3 * n:] == 7.0).all()


def test_async_pack_from_one_arena(dev):
    """w, m, v and the snapshot carved one after another from one allocation
    ([w | m | v | snapshot]): adjacent but disjoint ranges are accepted, and an
    overlapping snapshot is refused."""
    n = 100_003
    A = torch.empty(6 * n, device=dev)
    w, m, v, snap = A[:n], A[n:2 * n], A[2 * n:3 * n], A[3 * n:]
    for x, seed in ((w, 1210), (m, 1211), (v, 1212)):
        x.copy_(workloads.custom(seed, n, 1.0, device=dev))
    nb = rcs.ckpt_bytes(n)
    ref, buf = (torch.empty(nb, dtype=torch.uint8, pin_memory=True) for _ in range(2))
    rcs.ckpt_pack(4, w, m, v, ref)
    copy_stream = torch.cuda.Stream()
    rcs.ckpt_pack_async(4, w, m, v, snap, buf, compute_stream=torch.cuda.current_stream(),
                        copy_stream=copy_stream)
    rcs.ckpt_pack_wait(snap)
    torch.cuda.synchronize()
    assert torch.equal(buf, ref)
    B = torch.empty(5 * n, device=dev)  # the snapshot's first third is v
    with pytest.raises(rcs.RcsError) as e:
        rcs.ckpt_pack_async(4, B[:n], B[n:2 * n], B[2 * n:3 * n], B[2 * n:], buf,
                            compute_stream=torch.cuda.current_stream(), copy_stream=copy_stream)
    assert e.value.status == rcs.EINVAL


def _unpacked(buf, n):
    raw = buf.numpy()
    return [torch.from_numpy(raw[8 + 4 * j * n: 8 + 4 * (j + 1) * n].view(np.float32).copy())
            for j in range(3)]


@pytest.mark.parametrize("n", [262_147, 1_000_000])
def test_native_writer_files_are_the_state_at_submit(dev, tmp_path, n):
    """The library's writer: each submit snapshots the state on the training
    stream while later updates go on; every file equals a synchronous pack
    taken at its step, keep=2 leaves the two newest, and a second wait
    reports nothing new."""
    wl = workloads.WORKLOADS["flat262k"]
    w = workloads.init_params(wl, device=dev, n=n)
    m, v = workloads.zeros_like_state(n, device=dev)
    g = torch.empty(n, device=dev)
    wr = rcs.CkptWriter(tmp_path, n, keep=2)
    ref, written = {}, []
    for t in range(1, 26):
        workloads.grads(wl, t, device=dev, n=n, out=g)
        rcs.adamw_clip_step(w, g, m, v, t, wl.lr, wl.wd, wl.clip)
        if t % 5 == 0:
            ref[t] = torch.empty(rcs.ckpt_bytes(n), dtype=torch.uint8, pin_memory=True)
            rcs.ckpt_pack(t, w, m, v, ref[t])
            if t > 5:
                written.append(wr.wait())
            wr.submit(t, w, m, v)
    written.append(wr.wait())
    assert wr.wait() == ""
    torch.cuda.synchronize()
    assert [os.path.basename(p) for p in written] == [rcs.step_file_name(t) for t in ref]
    assert sorted(os.listdir(tmp_path)) == ["step_000020.bin", "step_000025.bin"]
    for t in (20, 25):
        assert open(tmp_path / rcs.step_file_name(t), "rb").read() == ref[t].numpy().tobytes()
    wr.close()


def test_native_writer_reports_a_failed_write(dev, tmp_path):
    n = 4099
    w = workloads.custom(300, n, 0.02, device=dev)
    m, v = workloads.zeros_like_state(n, device=dev)
    d = tmp_path / "ckpt"
    wr = rcs.CkptWriter(d, n, keep=1)
    os.rmdir(d)  # the directory is gone: the worker's write fails
    wr.submit(1, w, m, v)
    with pytest.raises(rcs.RcsError) as e:
        wr.wait()
    assert e.value.status == rcs.EIO
    assert wr.wait() == ""  # reported once
    wr.submit(2, w, m, v)  # fails in the background again ...
    with pytest.raises(rcs.RcsError) as e:
        # ... and a later submit reports it, submitting nothing: at the latest the
        # one that reuses step 2's host image, which waits for step 2's write
        for step in (3, 4):
            wr.submit(step, w, m, v)
    assert e.value.status == rcs.EIO
    try:
        wr.wait()  # step 3's write, if it went out, failed too
    except rcs.RcsError as e3:
        assert e3.status == rcs.EIO
    assert wr.wait() == ""
    os.makedirs(d)
    wr.submit(4, w, m, v)
    assert os.path.basename(wr.wait()) == "step_000004.bin"
    assert os.listdir(d) == ["step_000004.bin"]
    wr.close()
    wr.close()  # idempotent


@pytest.mark.parametrize("mode", ["sync", "async"])
def test_signal_driven_step_files_resume_bit_identical(dev, tmp_path, mode):
    """A child trains, gets SIGUSR1 after step 30 (writes, continues) and
    SIGTERM after step 70 (writes, exits); a second child resumes from the
    newest file and finishes 100 steps. Its final state equals a straight run
    byte for byte."""
    wl, n, total = "flat262k", 262_144, 100
    env = dict(os.environ)
    cmd = [sys.executable, "-u", os.path.join(HERE, "resume_child.py"), str(tmp_path), wl,
           str(n), str(total)]
    tail = [mode] if mode == "async" else []
    r1 = subprocess.run(cmd + ["30", "70"] + tail, capture_output=True, text=True, timeout=240,
                        env=env)
    print(r1.stdout, r1.stderr[-2000:])
    assert r1.returncode == 0
    assert "SIGTERM after step 70" in r1.stdout
    names = sorted(os.listdir(tmp_path))
    assert names == ["step_000030.bin", "step_000070.bin"], names
    r2 = subprocess.run(cmd + ["0", "0"] + tail, capture_output=True, text=True, timeout=240,
                        env=env)
    print(r2.stdout, r2.stderr[-2000:])
    assert r2.returncode == 0 and "resumed at step 70" in r2.stdout
    final = open(tmp_path / "step_000100.bin", "rb").read()
    # straight run in this process
    W = workloads.WORKLOADS[wl]
    w = workloads.init_params(W, device=dev, n=n)
    m, v = workloads.zeros_like_state(n, device=dev)
    g = torch.empty(n, device=dev)
    for t in range(1, total + 1):
        workloads.grads(W, t, device=dev, n=n, out=g)
        rcs.adamw_clip_step(w, g, m, v, t, W.lr, W.wd, W.clip)
    buf = torch.empty(rcs.ckpt_bytes(n), dtype=torch.uint8, pin_memory=True)
    rcs.ckpt_pack(total, w, m, v, buf)
    torch.cuda.synchronize()
    assert buf.numpy().tobytes() == final


def test_resume_after_sigkill_redoes_the_lost_updates(dev, tmp_path):
    """A crash between checkpoints: the child writes a step file every 25
    updates, finishes update 60 and is killed with SIGKILL (while it waits on
    the host, no device work or write in flight). A second child resumes from
    the newest valid file (step 50), redoes 51-60 and runs to 100; its final
    file is byte-identical to a straight run's."""
    wl, n, total = "flat262k", 262_144, 100
    cmd = [sys.executable, "-u", os.path.join(HERE, "resume_child.py"), str(tmp_path), wl,
           str(n), str(total), "0", "0", "sync", "25"]
    p = subprocess.Popen(cmd + ["60"], stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                         text=True)
    stalled = False
    try:
        for line in p.stdout:
            print(line, end="")
            if "stalled after step 60" in line:
                stalled = True
                break
    finally:
        p.kill()
        p.wait(timeout=60)
    assert stalled, p.stderr.read()[-2000:]
    assert p.returncode == -9
    assert sorted(os.listdir(tmp_path)) == ["step_000025.bin", "step_000050.bin"]
    r2 = subprocess.run(cmd + ["0"], capture_output=True, text=True, timeout=240)
    print(r2.stdout, r2.stderr[-2000:])
    assert r2.returncode == 0 and "resumed at step 50" in r2.stdout
    final = open(tmp_path / "step_000100.bin", "rb").read()
    W = workloads.WORKLOADS[wl]
    w = workloads.init_params(W, device=dev, n=n)
    m, v = workloads.zeros_like_state(n, device=dev)
    g = torch.empty(n, device=dev)
    for t in range(1, total + 1):
        workloads.grads(W, t, device=dev, n=n, out=g)
        rcs.adamw_clip_step(w, g, m, v, t, W.lr, W.wd, W.clip)
    buf = torch.empty(rcs.ckpt_bytes(n), dtype=torch.uint8, pin_memory=True)
    rcs.ckpt_pack(total, w, m, v, buf)
    torch.cuda.synchronize()
    assert buf.numpy().tobytes() == final


def test_weights_only_resume_diverges(dev):
    """Why m and v are in the file: resuming from the weights alone (m = v = 0,
    t restarted at 1) takes a different trajectory from the full resume,
    which is byte-identical to the straight run."""
    wl = workloads.WORKLOADS["flat262k"]
    n, k, total = wl.n, 40, 50
    w = workloads.init_params(wl, device=dev)
    m, v = workloads.zeros_like_state(n, device=dev)
    g = torch.empty(n, device=dev)
    for t in range(1, k + 1):
        workloads.grads(wl, t, device=dev, out=g)
        rcs.adamw_clip_step(w, g, m, v, t, wl.lr, wl.wd, wl.clip)
    full = [w.clone(), m.clone(), v.clone()]
    weights_only = [w.clone(), torch.zeros_like(m), torch.zeros_like(v)]
    for t in range(k + 1, total + 1):
        workloads.grads(wl, t, device=dev, out=g)
        rcs.adamw_clip_step(full[0], g, full[1], full[2], t, wl.lr, wl.wd, wl.clip)
        rcs.adamw_clip_step(weights_only[0], g, weights_only[1], weights_only[2], t - k,
                            wl.lr, wl.wd, wl.clip)
    torch.cuda.synchronize()
    diff = (full[0] - weights_only[0]).abs().max().item()
    assert diff > 10 * wl.lr, diff  # the first restarted step alone moves w by about lr
