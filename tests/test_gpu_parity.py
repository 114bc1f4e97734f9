"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar (from the method's precision): the float64 pre-clip norm within 1e-12
relative; w, m, v within 2 float32 ulp per element after every step (the
float32 op sequence is the same on both sides, so they are expected to be
bit-identical unless the two float64 norms round the clip factor apart);
headers, layout and packed bytes bit-exact; a packed-and-resumed run
bit-identical to the straight run.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
import resumable_checkpoint_state_amd as rcs
import workloads
from util import bits, max_ulp

pytestmark = pytest.mark.gpu

NORM_RTOL = 1e-12
ULP_TOL = 2


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rcs.lib()
    torch.cuda.set_device(0)
    return torch.device("cuda:0")


def _host(t):
    return t.detach().cpu().numpy()


def _gpu_norm():
    return float(rcs.last_grad_norm().cpu())


def _check_state(w, m, v, ow, om, ov, ctx):
    for name, a, b in (("w", w, ow), ("m", m, om), ("v", v, ov)):
        d = max_ulp(_host(a), b)
        assert d <= ULP_TOL, f"{ctx}: {name} max ulp distance {d}"


# ---------------------------------------------------------------- device arithmetic

def _fp32_div_sqrt(a, b):
    """q = a / b, r = sqrtf(a) on the device, from the tests' probe library
    (tests/native/fp32_probe.hip, built by __graft_entry__.build())."""
    path = os.path.join(os.path.dirname(__file__), "native", "libfp32probe.so")
    L = ctypes.CDLL(path)
    L.fp32_div_sqrt_probe.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_void_p]
    L.fp32_div_sqrt_probe.restype = ctypes.c_int
    q, r = torch.empty_like(a), torch.empty_like(a)
    assert L.fp32_div_sqrt_probe(a.data_ptr(), b.data_ptr(), q.data_ptr(), r.data_ptr(),
                                 a.numel(), torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    return q, r


def test_fp32_divide_and_sqrt_are_correctly_rounded(dev):
    rng = np.random.default_rng(0)
    n = 1 << 20
    a = rng.standard_normal(n).astype(np.float32) * np.float32(1e3)
    b = rng.standard_normal(n).astype(np.float32)
    e = rng.integers(-149, 127, n)
    a[: n // 4] = np.ldexp(rng.random(n // 4) + 0.5, e[: n // 4]).astype(np.float32)
    b[n // 4: n // 2] = np.ldexp(rng.random(n // 4) + 0.5, e[n // 4: n // 2]).astype(np.float32)
    a[:64] = np.float32(1.4e-45) * np.arange(1, 65, dtype=np.float32)  # subnormal numerators
    b[b == 0] = 1.0
    q, r = _fp32_div_sqrt(torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev))
    with np.errstate(all="ignore"):
        q_ref = a / b
        r_ref = np.sqrt(np.abs(a))
    assert (bits(_host(q)) == bits(q_ref)).all()
    pos = a >= 0
    assert (bits(_host(r))[pos] == bits(r_ref)[pos]).all()


# ---------------------------------------------------------------- norm

@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 63, 64, 65, 1023, 4096, 4097, 16387, 262_147,
                               1_000_003, 40_000_003])
def test_norm_parity_sizes(dev, n):
    g = workloads.custom(100, n, 0.01, device=dev)
    out = rcs.grad_global_norm(g)
    torch.cuda.synchronize()
    ref = oracle.grad_norm(_host(g))
    got = float(out.cpu())
    assert abs(got - ref) <= NORM_RTOL * ref, (n, got, ref)


# (elements past a 512-byte allocation start, n): heads of 63, 62, 61, 47 and 1
# elements before g's next 256-byte boundary; 16-byte heads when fewer than 4
# elements would follow it (n = 66: head 3, body 63); the scalar loop when even
# that leaves fewer than 4 (n = 6); several grid-stride passes with the
# cache-allocating tail (n = 40,000,003).
@pytest.mark.parametrize("offset,n", [(1, 100_003), (2, 100_003), (3, 100_003), (17, 100_003),
                                      (63, 100_003), (1, 66), (1, 67), (1, 6),
                                      (2, 40_000_003)])
def test_norm_parity_unaligned(dev, offset, n):
    base = workloads.custom(101, n + offset, 1.0, device=dev)
    g = base[offset:]
    out = rcs.grad_global_norm(g)
    torch.cuda.synchronize()
    ref = oracle.grad_norm(_host(g).copy())
    assert abs(float(out.cpu()) - ref) <= NORM_RTOL * ref


def test_norm_exact_power_of_two_cases(dev):
    n = 1 << 18
    g = torch.full((n,), 2.0 ** -6, device=dev)
    assert float(rcs.grad_global_norm(g).cpu()) == 8.0
    g.fill_(2.0 ** -10)
    assert float(rcs.grad_global_norm(g).cpu()) == 0.5
    g.zero_()
    g[12345] = -3.25
    assert float(rcs.grad_global_norm(g).cpu()) == 3.25
    g.zero_()
    assert float(rcs.grad_global_norm(g).cpu()) == 0.0


def test_norm_into_pinned_host(dev):
    g = workloads.custom(102, 70_001, 1.0, device=dev)
    out = torch.zeros(1, dtype=torch.float64, pin_memory=True)
    rcs.grad_global_norm(g, out=out)
    torch.cuda.synchronize()
    ref = oracle.grad_norm(_host(g))
    assert abs(float(out[0]) - ref) <= NORM_RTOL * ref


def test_clip_exact_power_of_two_update(dev):
    """n = 2^18, g = 2^-6: norm 8, s = 0.125 exactly on both sides, so the
    whole update must be bit-identical."""
    n = 1 << 18
    w = workloads.custom(103, n, 0.02, device=dev)
    g = torch.full((n,), 2.0 ** -6, device=dev)
    m, v = workloads.zeros_like_state(n, device=dev)
    ow, om, ov = _host(w).copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    rcs.adamw_clip_step(w, g, m, v, 1, 3e-3, 0.01, 1.0)
    oracle.adamw_clip_step(ow, _host(g), om, ov, 1, 3e-3, 0.01, 1.0)
    torch.cuda.synchronize()
    assert _gpu_norm() == 8.0
    for a, b in ((w, ow), (m, om), (v, ov)):
        assert (bits(_host(a)) == bits(b)).all()


# ---------------------------------------------------------------- update

def _run_parity(dev, wl, steps, n=None, scale=1.0):
    n = wl.n if n is None else n
    w = workloads.init_params(wl, device=dev, n=n)
    m, v = workloads.zeros_like_state(n, device=dev)
    ow, om, ov = _host(w).copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    g = torch.empty(n, device=dev)
    diffs = 0
    for t in range(1, steps + 1):
        workloads.grads(wl, t, device=dev, n=n, out=g)
        if scale != 1.0:
            g.mul_(scale)
        rcs.adamw_clip_step(w, g, m, v, t, wl.lr, wl.wd, wl.clip)
        gn = _gpu_norm()
        rc, on = oracle.adamw_clip_step(ow, _host(g), om, ov, t, wl.lr, wl.wd, wl.clip)
        assert rc == oracle.OK
        assert abs(gn - on) <= NORM_RTOL * on, (t, gn, on)
        _check_state(w, m, v, ow, om, ov, f"{wl.name} n={n} t={t}")
        diffs += int((bits(_host(w)) != bits(ow)).sum())
    return w, m, v, diffs


def test_update_parity_flat262k_all_80_steps(dev):
    wl = workloads.WORKLOADS["flat262k"]
    _, _, _, diffs = _run_parity(dev, wl, wl.steps)
    print(f"flat262k: {diffs} w elements off by 1-2 ulp over {wl.steps} steps")


@pytest.mark.parametrize("n", [1, 3, 5, 511, 513, 4099, 65_537])
def test_update_parity_ragged_sizes(dev, n):
    wl = workloads.WORKLOADS["flat262k"]
    _run_parity(dev, wl, 3, n=n, scale=50.0)


# (offsets of w, g, m, v in elements past a 512-byte allocation start, n).
# Offsets equal modulo 4 take the vector kernels: the head runs to w's next
# 256-byte boundary (64 - offset elements: bodies of exactly 4 and 7 behind a
# 63-element head, head and tail in one block), or to the next 16-byte one when
# fewer than 4 elements would follow (heads of 1-3, bodies of 4, 5 and 7); g, m
# and v may sit at other 256-byte phases (1, 5, 9, 65). The anchor is w or m,
# whichever shares its 128-byte line phase with more of the written arrays (m
# only when v shares its 16-byte phase). Arrays whose offset differs from the
# anchor's modulo 4 take shifted 16-byte vectors in the vector kernels
# (adamw_update_mixed: every reachable combination appears here, in both
# final-reduction forms); arrays at the anchor's 16-byte but another line
# phase take aligned vectors with cache-retaining accesses on the lines two
# waves share. Views
# too short for either head take the scalar kernels.
UNALIGNED_CASES = [((1, 1, 1, 1), 50_001), ((2, 2, 2, 2), 50_001), ((3, 3, 3, 3), 50_001),
                   ((1, 1, 1, 1), 67), ((1, 1, 1, 1), 70), ((2, 2, 2, 2), 66),
                   ((3, 3, 3, 3), 5), ((3, 3, 3, 3), 6), ((1, 1, 1, 1), 7), ((2, 2, 2, 2), 9),
                   ((1, 5, 9, 65), 50_001), ((4, 8, 12, 0), 4099),
                   ((1, 1, 1, 1), 8_388_611), ((3, 3, 3, 3), 8_388_608),
                   ((1, 2, 1, 1), 50_001), ((0, 3, 0, 0), 12_800_003), ((2, 0, 2, 2), 67),
                   ((3, 1, 3, 3), 8_388_611), ((1, 0, 1, 1), 8_388_608),
                   ((1, 2, 0, 3), 50_001), ((0, 0, 0, 1), 4099), ((1, 0, 0, 0), 50_001),
                   ((0, 1, 2, 3), 8_388_608), ((3, 3, 0, 3), 12_800_003), ((2, 2, 2, 0), 66),
                   ((1, 1, 2, 1), 70), ((1, 1, 0, 2), 50_001), ((1, 0, 1, 2), 4099),
                   ((3, 0, 1, 3), 12_800_003), ((2, 2, 2, 2), 5),
                   # m and v sharing a phase w does not: the body is anchored on m
                   # and w takes the shifted vectors (a 1-vector body with a tail too)
                   ((1, 2, 0, 0), 50_001), ((1, 2, 0, 0), 12_800_003), ((1, 0, 0, 0), 8_388_611),
                   ((1, 0, 0, 0), 6), ((2, 0, 0, 0), 5), ((0, 1, 2, 0), 4099),
                   ((0, 0, 0, 1), 12_800_003), ((1, 1, 0, 2), 8_388_611),
                   ((1, 0, 1, 2), 12_800_003), ((0, 1, 2, 3), 12_800_003),
                   # line phases: w 16 bytes past the others (anchored on m), the
                   # written arrays split 2 + 1 or 1 + 1 + 1 over line phases, g
                   # alone off them, with fold and without, ragged tails
                   ((4, 0, 0, 0), 50_001), ((4, 0, 0, 0), 12_800_003), ((4, 4, 0, 0), 8_388_611),
                   ((0, 0, 4, 4), 8_388_608), ((0, 0, 0, 4), 12_800_003), ((0, 4, 0, 0), 4099),
                   ((8, 0, 4, 12), 50_001), ((0, 0, 28, 28), 70), ((28, 0, 0, 0), 66),
                   ((5, 1, 1, 1), 50_001), ((1, 5, 2, 2), 12_800_003), ((4, 0, 0, 1), 8_388_611)]


@pytest.mark.parametrize("offs,n", UNALIGNED_CASES)
def test_update_parity_unaligned_views(dev, offs, n):
    wl = workloads.WORKLOADS["flat262k"]
    W, G, M, V = (torch.zeros(n + o, device=dev) for o in offs)
    w, g, m, v = (X[o:] for X, o in zip((W, G, M, V), offs))
    w.copy_(workloads.init_params(wl, device=dev, n=n))
    ow, om, ov = _host(w).copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in (1, 2, 3):
        g.copy_(workloads.grads(wl, t, device=dev, n=n)).mul_(10.0)
        rcs.adamw_clip_step(w, g, m, v, t, wl.lr, wl.wd, wl.clip)
        gn = _gpu_norm()
        rc, on = oracle.adamw_clip_step(ow, _host(g).copy(), om, ov, t, wl.lr, wl.wd, wl.clip)
        assert rc == oracle.OK and abs(gn - on) <= NORM_RTOL * on, (offs, n, t, gn, on)
        _check_state(w, m, v, ow, om, ov, f"offsets={offs} n={n} t={t}")
    # the elements just outside the views are never written
    for X, o in zip((W, G, M, V), offs):
        assert (X[:o] == 0).all()


def test_update_parity_andrea12m(dev):
    _run_parity(dev, workloads.WORKLOADS["andrea12m"], 3)


def test_update_parity_andrea12m_both_clip_branches(dev):
    """Steps 1, 2 stay under the threshold (s = 1, g used as is); step 3 has
    the outliers and clips."""
    wl = workloads.WORKLOADS["andrea12m_b"]
    n = wl.n
    w = workloads.init_params(wl, device=dev)
    m, v = workloads.zeros_like_state(n, device=dev)
    ow, om, ov = _host(w).copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    norms = []
    for t in (1, 2, 3):
        g = workloads.grads(wl, t, device=dev)
        rcs.adamw_clip_step(w, g, m, v, t, wl.lr, wl.wd, wl.clip)
        _, on = oracle.adamw_clip_step(ow, _host(g), om, ov, t, wl.lr, wl.wd, wl.clip)
        norms.append(on)
        assert abs(_gpu_norm() - on) <= NORM_RTOL * on
        _check_state(w, m, v, ow, om, ov, f"andrea12m_b t={t}")
    assert norms[0] < wl.clip and norms[1] < wl.clip and norms[2] > wl.clip


def test_update_parity_andrea120m_full_size(dev):
    _run_parity(dev, workloads.WORKLOADS["andrea120m"], 2)


def test_update_parity_stress_subnormals_full_size(dev):
    wl = workloads.WORKLOADS["andrea120m_stress"]
    w, m, v, _ = _run_parity(dev, wl, 2)
    mh = _host(m)
    sub = (mh != 0) & (np.abs(mh) < np.float32(1.1754944e-38))
    assert sub.sum() > 0, "stress grads should leave subnormal first moments"


# With 16-byte aligned arrays and n up to 8,388,608 the update kernel reduces
# the norm partials itself instead of a separate final kernel; its reduction
# must give the final kernel's bits. grad_global_norm always runs the final
# kernel, so the two norms of one gradient must be equal (sizes from one
# partial to the 256-block cap, both sides of the fold limit, ragged tails).
@pytest.mark.parametrize("n", [4, 5, 4099, 262_147, 2_097_152, 2_097_153, 8_388_608, 8_388_611,
                               33_554_435])
def test_step_norm_same_bits_as_final_kernel(dev, n):
    g = workloads.custom(140, n, 0.01, device=dev)
    g[n // 2] = 3.0  # one large element: the step clips
    w = workloads.custom(141, n, 0.02, device=dev)
    m, v = workloads.zeros_like_state(n, device=dev)
    ow, og = _host(w).copy(), _host(g)
    om, ov = np.zeros(n, np.float32), np.zeros(n, np.float32)
    standalone = float(rcs.grad_global_norm(g).cpu())
    for t in (1, 2):
        rcs.adamw_clip_step(w, g, m, v, t, 3e-3, 0.01, 1.0)
        step = _gpu_norm()
        assert np.float64(step).tobytes() == np.float64(standalone).tobytes(), (n, step, standalone)
        rc, on = oracle.adamw_clip_step(ow, og, om, ov, t, 3e-3, 0.01, 1.0)
        assert rc == oracle.OK and on > 1.0
        assert abs(step - on) <= NORM_RTOL * on
        _check_state(w, m, v, ow, om, ov, f"n={n} t={t}")


@pytest.mark.parametrize("n,off,goff", [(10_000, 0, 0), (5_000_001, 0, 0), (10_000, 1, 1),
                                         (10_000, 1, 2), (9_000_001, 0, 3), (3, 0, 0)])
def test_nonfinite_norm_skips_update(dev, n, off, goff):
    """Every update form skips: the vector kernels (equal offsets, with and
    without a peeled head, both final-reduction forms; g at another phase than
    w, m, v) and the scalar one after the final kernel (n < 4)."""
    w = workloads.custom(104, n + off, 0.02, device=dev)[off:]
    m = workloads.custom(105, n + off, 0.01, device=dev)[off:]
    v = workloads.custom(106, n + off, 0.01, device=dev)[off:].abs_()
    before = [_host(x).copy() for x in (w, m, v)]
    for bad in (float("inf"), float("nan")):
        g = workloads.custom(107, n + goff, 1.0, device=dev)[goff:]
        g[min(777, n - 1)] = bad
        rcs.adamw_clip_step(w, g, m, v, 4, 3e-3, 0.01, 1.0)
        norm = _gpu_norm()
        assert not np.isfinite(norm)
        for x, b in zip((w, m, v), before):
            assert (bits(_host(x)) == bits(b)).all()


# ---------------------------------------------------------------- pack / resume

def _pinned(nbytes):
    return torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)


def test_pack_bytes_match_oracle_layout(dev):
    n = 262_147
    w = workloads.custom(108, n, 1.0, device=dev)
    m = workloads.custom(109, n, 1.0, device=dev)
    v = workloads.custom(110, n, 1.0, device=dev)
    buf = _pinned(rcs.ckpt_bytes(n))
    rcs.ckpt_pack(80, w, m, v, buf)
    torch.cuda.synchronize()
    _, ob = oracle.ckpt_pack(80, _host(w), _host(m), _host(v))
    assert buf.numpy().tobytes() == ob.tobytes()


def test_unpack_rejects_and_leaves_device_untouched(dev):
    n = 1000
    w = workloads.custom(111, n, 1.0, device=dev)
    keep = _host(w).copy()
    buf = _pinned(rcs.ckpt_bytes(n))
    rcs.ckpt_pack(3, w, w.clone(), w.clone(), buf)
    torch.cuda.synchronize()
    bad = torch.cat([buf, torch.zeros(1, dtype=torch.uint8)])
    m2, v2 = torch.zeros_like(w), torch.zeros_like(w)
    with pytest.raises(rcs.RcsError):
        rcs.ckpt_unpack(bad, w, m2, v2)
    with pytest.raises(rcs.RcsError):
        rcs.ckpt_unpack(buf[:-1].clone(), w, m2, v2)
    with pytest.raises(rcs.RcsError):
        rcs.ckpt_unpack(buf, w[:-1], m2[:-1], v2[:-1])
    torch.cuda.synchronize()
    assert (bits(_host(w)) == bits(keep)).all() and not m2.any() and not v2.any()


def _straight_vs_resumed(dev, wl, steps, pack_at, n=None):
    n = wl.n if n is None else n
    w0 = workloads.init_params(wl, device=dev, n=n)
    g = torch.empty(n, device=dev)
    # straight
    w, (m, v) = w0.clone(), workloads.zeros_like_state(n, device=dev)
    for t in range(1, steps + 1):
        workloads.grads(wl, t, device=dev, n=n, out=g)
        rcs.adamw_clip_step(w, g, m, v, t, wl.lr, wl.wd, wl.clip)
    # run to pack_at, pack, drop the state, unpack into fresh buffers, resume
    w2, (m2, v2) = w0.clone(), workloads.zeros_like_state(n, device=dev)
    for t in range(1, pack_at + 1):
        workloads.grads(wl, t, device=dev, n=n, out=g)
        rcs.adamw_clip_step(w2, g, m2, v2, t, wl.lr, wl.wd, wl.clip)
    buf = _pinned(rcs.ckpt_bytes(n))
    rcs.ckpt_pack(pack_at, w2, m2, v2, buf)
    torch.cuda.synchronize()
    del w2, m2, v2
    w3, m3, v3 = (torch.full((n,), float("nan"), device=dev) for _ in range(3))
    step = rcs.ckpt_unpack(buf, w3, m3, v3)
    assert step == pack_at
    for t in range(step + 1, steps + 1):
        workloads.grads(wl, t, device=dev, n=n, out=g)
        rcs.adamw_clip_step(w3, g, m3, v3, t, wl.lr, wl.wd, wl.clip)
    out_a, out_b = _pinned(rcs.ckpt_bytes(n)), _pinned(rcs.ckpt_bytes(n))
    rcs.ckpt_pack(steps, w, m, v, out_a)
    rcs.ckpt_pack(steps, w3, m3, v3, out_b)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b), f"{wl.name}: resumed state differs from straight run"
    return w, m, v, out_a


def test_resume_bit_identical_flat262k(dev):
    wl = workloads.WORKLOADS["flat262k"]
    w, m, v, packed = _straight_vs_resumed(dev, wl, wl.steps, 40)
    # the packed step_000080.bin: header and size fixed by the layout
    assert packed.numel() == 3_145_736
    rc, step, n = oracle.ckpt_header(packed.numpy())
    assert (rc, step, n) == (oracle.OK, 80, wl.n)
    # and the GPU trajectory stays within the bar of the oracle's
    ow = _host(workloads.init_params(wl, device=dev)).copy()
    om, ov = np.zeros(wl.n, np.float32), np.zeros(wl.n, np.float32)
    for t in range(1, wl.steps + 1):
        oracle.adamw_clip_step(ow, _host(workloads.grads(wl, t, device=dev)), om, ov, t,
                               wl.lr, wl.wd, wl.clip)
    _check_state(w, m, v, ow, om, ov, "flat262k after 80 steps")


@pytest.mark.parametrize("lost", ["moments", "step_count"])
def test_resume_without_the_full_state_differs(dev, lost):
    """Each piece of the state besides w on its own (test_gpu_next drops both
    at once): resuming flat262k at step 40 without the moments (m = v = 0) or
    with the update counter restarted at 1 (bias corrections of a fresh run)
    leaves a final w measurably off the straight run's, so the resume tests
    would notice a pack that dropped either."""
    wl = workloads.WORKLOADS["flat262k"]
    n, steps, pack_at = wl.n, wl.steps, 40
    w0 = workloads.init_params(wl, device=dev)
    g = torch.empty(n, device=dev)
    w, (m, v) = w0.clone(), workloads.zeros_like_state(n, device=dev)
    for t in range(1, pack_at + 1):
        workloads.grads(wl, t, device=dev, out=g)
        rcs.adamw_clip_step(w, g, m, v, t, wl.lr, wl.wd, wl.clip)
    w2, m2, v2 = w.clone(), m.clone(), v.clone()
    if lost == "moments":
        m2.zero_()
        v2.zero_()
    for t in range(pack_at + 1, steps + 1):
        workloads.grads(wl, t, device=dev, out=g)
        rcs.adamw_clip_step(w, g, m, v, t, wl.lr, wl.wd, wl.clip)
        t2 = t if lost == "moments" else t - pack_at
        rcs.adamw_clip_step(w2, g, m2, v2, t2, wl.lr, wl.wd, wl.clip)
    torch.cuda.synchronize()
    diff = float((w - w2).abs().max())
    assert diff > 1e-4, (lost, diff)


def test_resume_bit_identical_andrea12m(dev):
    """ANDREA-12M's cadence: 200 updates, resumed from the step-100 pack."""
    wl = workloads.WORKLOADS["andrea12m"]
    _, _, _, packed = _straight_vs_resumed(dev, wl, wl.steps, 100)
    assert packed.numel() == 153_600_008


def test_resume_bit_identical_stress_full_size(dev):
    wl = workloads.WORKLOADS["andrea120m_stress"]
    _, _, _, packed = _straight_vs_resumed(dev, wl, wl.steps, 100)
    assert packed.numel() == 1_492_282_376


# ---------------------------------------------------------------- near the int32 limit

@pytest.mark.timeout(800)
def test_flat2e9_all_10_steps_sampled_parity_and_pack(dev):
    """n = 2e9 (32 GB of w, g, m, v) as configured: all 10 updates in the
    launch configuration the benchmark times. Every step the float64 norm is
    checked against the oracle's norm streamed over all 2e9 gradients, and 14
    sampled 1 Mi-element chunks (the first and the last included) are carried
    through the oracle's elementwise update with the clip factor from that
    streamed norm; w, m, v on them within 2 ulp after every step. Then one
    24 GB pack after step 10: header and sampled byte ranges, and an unpack
    into fresh arrays that restores w, m, v bit for bit."""
    wl = workloads.WORKLOADS["flat2e9"]
    n = wl.n
    chunk = 1 << 20
    offs = sorted({0, n - chunk, *[int(k * (n - chunk) // 13) for k in range(1, 13)]})
    print(f"flat2e9: n={n}, {len(offs)} sampled chunks", flush=True)
    w = workloads.init_params(wl, device=dev)
    m, v = workloads.zeros_like_state(n, device=dev)
    g = torch.empty(n, device=dev)
    state = {o: [_host(x[o:o + chunk]).copy() for x in (w, m, v)] for o in offs}
    for t in range(1, wl.steps + 1):
        workloads.grads(wl, t, device=dev, out=g)
        gs = {o: _host(g[o:o + chunk]).copy() for o in offs}
        rcs.adamw_clip_step(w, g, m, v, t, wl.lr, wl.wd, wl.clip)
        gpu_norm = _gpu_norm()
        acc = oracle.NormAccumulator()
        for lo in range(0, n, 1 << 28):
            acc.add(_host(g[lo:min(lo + (1 << 28), n)]))
        onorm = acc.norm()
        print(f"flat2e9 t={t}: norm gpu {gpu_norm!r} oracle {onorm!r}", flush=True)
        assert abs(gpu_norm - onorm) <= NORM_RTOL * onorm
        s = oracle.clip_scale(onorm, wl.clip)
        bc1, bc2, decay = oracle.scalars(t, wl.lr, wl.wd)
        for o in offs:
            ow, om, ov = state[o]
            oracle.adamw_elems(ow, gs[o], om, ov, float(s), float(bc1), float(bc2), float(decay),
                               wl.lr)
            _check_state(w[o:o + chunk], m[o:o + chunk], v[o:o + chunk], ow, om, ov,
                         f"flat2e9 t={t} chunk at {o}")
    del g
    nb = rcs.ckpt_bytes(n)
    assert nb == 24_000_000_008
    buf = _pinned(nb)
    rcs.ckpt_pack(wl.steps, w, m, v, buf)
    torch.cuda.synchronize()
    raw = buf.numpy()
    assert oracle.ckpt_header(raw[:8].copy()) == (oracle.OK, wl.steps, n)
    for o in offs:
        for k, x in enumerate((w, m, v)):
            lo = 8 + 4 * k * n + 4 * o
            assert raw[lo:lo + 4 * chunk].tobytes() == _host(x[o:o + chunk]).tobytes()
    w2, m2, v2 = (torch.empty(n, device=dev) for _ in range(3))
    assert rcs.ckpt_unpack(buf, w2, m2, v2) == wl.steps
    torch.cuda.synchronize()
    for a, b in ((w, w2), (m, m2), (v, v2)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


# ---------------------------------------------------------------- whole runs at full size

def _full_run(dev, wl, check_every, resume_at=None):
    """All wl.steps updates on the GPU beside the oracle's straight run: the
    norm within 1e-12 every step, w, m, v within 2 ulp every check_every steps
    and at every pack, packed bytes equal to the oracle's pack of its own state
    whenever the two states are bit-identical. resume_at: at that step the GPU
    state is packed, the device arrays dropped, fresh NaN-filled ones unpacked
    from the bytes, and the run continues from them (t = step + 1) while the
    oracle goes straight on, so every later check compares a resumed GPU run
    with a run that never stopped."""
    n = wl.n
    w = workloads.init_params(wl, device=dev)
    m, v = workloads.zeros_like_state(n, device=dev)
    ow, om, ov = _host(w).copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    g = torch.empty(n, device=dev)
    worst = 0
    t = 0
    while t < wl.steps:
        t += 1
        workloads.grads(wl, t, device=dev, n=n, out=g)
        rcs.adamw_clip_step(w, g, m, v, t, wl.lr, wl.wd, wl.clip)
        gn = _gpu_norm()
        rc, on = oracle.adamw_clip_step(ow, _host(g), om, ov, t, wl.lr, wl.wd, wl.clip)
        assert rc == oracle.OK and abs(gn - on) <= NORM_RTOL * on, (t, gn, on)
        packing = t in wl.pack_at or t == resume_at
        if t % check_every == 0 or t == wl.steps or packing:
            for name, a, b in (("w", w, ow), ("m", m, om), ("v", v, ov)):
                d = max_ulp(_host(a), b)
                worst = max(worst, d)
                assert d <= ULP_TOL, f"{wl.name} t={t}: {name} max ulp distance {d}"
            print(f"{wl.name}: step {t} within {worst} ulp", flush=True)
        if packing:
            buf = _pinned(rcs.ckpt_bytes(n))
            rcs.ckpt_pack(t, w, m, v, buf)
            torch.cuda.synchronize()
            assert oracle.ckpt_header(buf.numpy()[:8].copy()) == (oracle.OK, t, n)
            if worst == 0:  # identical states pack to identical bytes
                _, ob = oracle.ckpt_pack(t, ow, om, ov)
                assert buf.numpy().tobytes() == ob.tobytes()
            if t == resume_at:
                del w, m, v
                w, m, v = (torch.full((n,), float("nan"), device=dev) for _ in range(3))
                t = rcs.ckpt_unpack(buf, w, m, v)
                assert t == resume_at
                print(f"{wl.name}: resumed from the step-{t} pack", flush=True)
    return worst


@pytest.mark.timeout(300)
def test_andrea12m_all_200_steps_against_oracle(dev):
    """ANDREA-12M as configured: 200 updates, a checkpoint every 100; the run
    resumes from its step-100 pack and its step-200 pack equals the oracle's."""
    wl = workloads.WORKLOADS["andrea12m"]
    print("andrea12m worst ulp:", _full_run(dev, wl, 20, resume_at=100))


@pytest.mark.timeout(600)
def test_andrea120m_all_100_steps_against_oracle(dev):
    wl = workloads.WORKLOADS["andrea120m"]
    print("andrea120m worst ulp:", _full_run(dev, wl, 25))


@pytest.mark.timeout(600)
def test_stress_all_200_steps_against_oracle_resumed_at_100(dev):
    """The subnormal-heavy stress workload as configured: 200 updates with
    gradients N(0, 1), 5% exact zeros and 0.1% near FLT_MIN (the clip fires
    every step, s ~ 9e-5, so g * s and the moments go subnormal), packed,
    dropped and unpacked at step 100, against the oracle's straight run."""
    wl = workloads.WORKLOADS["andrea120m_stress"]
    print("stress worst ulp:", _full_run(dev, wl, 25, resume_at=100))


@pytest.mark.timeout(600)
def test_max_n_int32_limit_ragged_tail(dev):
    """n = 2^31 - 1, the largest n the int32 header can hold (n % 4 == 3, so
    the vector kernels end in a 3-element scalar tail): one update, norm
    against the oracle's streamed norm, w, m, v on the first, a middle and the
    last 1 Mi elements; then the in-place clip of the same g (same norm, g * s
    on those chunks) and grad_zero (the chunks and the last 3 elements)."""
    n = rcs.MAX_N
    wl = workloads.WORKLOADS["flat2e9"]
    chunk = 1 << 20
    offs = [0, (n // 2) // 4 * 4 + 1, n - chunk]
    w = workloads.custom(300, n, 0.02, device=dev)
    g = workloads.custom(301, n, 1e-4, device=dev)
    m = workloads.custom(302, n, 1e-5, device=dev)
    v = workloads.custom(303, n, 1e-6, device=dev).square_()
    before = {o: [_host(x[o:o + chunk]).copy() for x in (w, g, m, v)] for o in offs}
    rcs.adamw_clip_step(w, g, m, v, 7, wl.lr, wl.wd, wl.clip)
    gpu_norm = _gpu_norm()
    acc = oracle.NormAccumulator()
    for lo in range(0, n, 1 << 28):
        acc.add(_host(g[lo:min(lo + (1 << 28), n)]))
    onorm = acc.norm()
    assert abs(gpu_norm - onorm) <= NORM_RTOL * onorm
    s = oracle.clip_scale(onorm, wl.clip)
    bc1, bc2, decay = oracle.scalars(7, wl.lr, wl.wd)
    for o in offs:
        ow, og, om, ov = before[o]
        oracle.adamw_elems(ow, og, om, ov, float(s), float(bc1), float(bc2), float(decay), wl.lr)
        _check_state(w[o:o + chunk], m[o:o + chunk], v[o:o + chunk], ow, om, ov,
                     f"max n chunk at {o}")
    # the in-place clip and the buffer reset at the same size (g is still the
    # gradient whose norm was just checked)
    rcs.grad_clip_inplace(g, wl.clip)
    assert _gpu_norm() == gpu_norm
    for o in offs:
        og = before[o][1].copy()
        oracle.scale_grads(og, float(s))  # g * s in float32, s from the full-length norm
        assert max_ulp(_host(g[o:o + chunk]), og) <= ULP_TOL, f"clip chunk at {o}"
    rcs.grad_zero(g)
    torch.cuda.synchronize()
    for o in offs:
        assert not bool(g[o:o + chunk].any()), f"grad_zero chunk at {o}"
    assert not bool(g[-3:].any())


@pytest.mark.parametrize("case", ["clip_inf", "lr_zero", "wd_zero", "t_max", "zero_grad",
                                  "inf_and_signed_zero_weights", "huge_grads", "tiny_lr"])
def test_edge_scalars_and_values(dev, case):
    n = 65_539
    t, lr, wd, clip = 3, 3e-3, 0.01, 1.0
    w = workloads.custom(400, n, 0.02, device=dev)
    g = workloads.custom(401, n, 0.05, device=dev)
    m = workloads.custom(402, n, 0.01, device=dev)
    v = workloads.custom(403, n, 0.01, device=dev).square_()
    if case == "clip_inf":
        clip = float("inf")
    elif case == "lr_zero":
        lr = 0.0
    elif case == "wd_zero":
        wd = 0.0
    elif case == "t_max":
        t = 2**31 - 1  # bias corrections round to 1.0f
    elif case == "zero_grad":
        g.zero_()
    elif case == "inf_and_signed_zero_weights":
        w[:8] = torch.tensor([float("inf"), float("-inf"), 0.0, -0.0] * 2)
    elif case == "huge_grads":
        g.fill_(3e38)  # float32 squares overflow, the float64 sum does not
    elif case == "tiny_lr":
        lr = 1e-30
    ow, og, om, ov = (_host(x).copy() for x in (w, g, m, v))
    rcs.adamw_clip_step(w, g, m, v, t, lr, wd, clip)
    gn = _gpu_norm()
    rc, on = oracle.adamw_clip_step(ow, og, om, ov, t, lr, wd, clip)
    assert rc == oracle.OK
    assert gn == on == 0.0 if case == "zero_grad" else abs(gn - on) <= NORM_RTOL * on
    _check_state(w, m, v, ow, om, ov, case)
    if case == "lr_zero":
        assert (_host(w) == _host(workloads.custom(400, n, 0.02, device=dev))).all()


def test_randomized_cases_against_oracle(dev):
    """160 seeded random cases, two updates each: sizes 1 .. ~70,000 (both
    launch forms, ragged tails), views 0-79 elements past an allocation's
    start (equal offsets modulo 4: vector kernels with a peeled head; else
    scalar), t up to
    2^31 - 2, lr, wd, clip and gradient scales over many decades (clipped and
    unclipped), micro-batch scales; the norm and w, m, v against the oracle at
    the usual bar."""
    rng = np.random.default_rng(20240607)
    clipped = unclipped = 0
    for case in range(160):
        n = int(np.exp(rng.uniform(0.0, np.log(70_000))))
        off = int(rng.choice([0, 0, 1, 2, 3, int(rng.integers(4, 80))]))
        offs = [off] * 4 if rng.random() < 0.8 else [int(x) for x in rng.integers(0, 80, 4)]
        t = int(min(np.exp(rng.uniform(0.0, np.log(2**31 - 2))), 2**31 - 2))
        lr = float(10 ** rng.uniform(-6, -1))
        wd = float(rng.choice([0.0, rng.uniform(0.0, 0.2)]))
        clip = float("inf") if rng.random() < 0.1 else float(10 ** rng.uniform(-3, 2))
        sigma = float(10 ** rng.uniform(-8, 1))
        scale = float(np.float32(1.0) / np.float32(rng.choice([1, 2, 3, 4, 7])))
        base = 1000 + 4 * case
        arrs = []
        for k, sd in enumerate((0.02, sigma, 0.01, 0.01)):
            x = workloads.custom(base + k, n + offs[k], sd, device=dev)[offs[k]:]
            arrs.append(x.square_() if k == 3 else x)
        w, g, m, v = arrs
        ow, og, om, ov = (_host(x).copy() for x in arrs)
        ctx = f"case {case}: n={n} offs={offs} t={t} lr={lr:.3g} wd={wd:.3g} clip={clip:.3g} " \
              f"sigma={sigma:.3g} scale={scale:.3g}"
        for tt in (t, t + 1):
            rcs.adamw_clip_step_accum(w, g, m, v, tt, lr, wd, clip, scale)
            gn = _gpu_norm()
            rc, on = oracle.adamw_clip_step_accum(ow, og, om, ov, tt, lr, wd, clip, scale)
            assert rc == oracle.OK, ctx
            assert abs(gn - on) <= NORM_RTOL * on, (ctx, gn, on)
            _check_state(w, m, v, ow, om, ov, ctx)
        clipped += on > clip
        unclipped += on <= clip
    assert clipped > 20 and unclipped > 20, (clipped, unclipped)


def test_two_streams_have_separate_workspaces(dev):
    """Two parameter sets updated concurrently on two streams: each stream has
    its own partials and clip scalars, so both match the oracle and each
    stream's last_grad_norm is its own."""
    n1, n2 = 1_000_003, 777_777
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    A = [workloads.custom(500 + k, n1, 0.02 if k == 0 else 0.0, device=dev) for k in range(3)]
    B = [workloads.custom(510 + k, n2, 0.02 if k == 0 else 0.0, device=dev) for k in range(3)]
    oA = [_host(x).copy() for x in A]
    oB = [_host(x).copy() for x in B]
    torch.cuda.synchronize()
    for t in (1, 2, 3):
        ga = workloads.custom(520 + t, n1, 0.05, device=dev)
        gb = workloads.custom(530 + t, n2, 0.5, device=dev)
        torch.cuda.synchronize()
        rcs.adamw_clip_step(A[0], ga, A[1], A[2], t, 3e-3, 0.01, 1.0, stream=sa)
        rcs.adamw_clip_step(B[0], gb, B[1], B[2], t, 1e-3, 0.1, 2.0, stream=sb)
        na = rcs.last_grad_norm(stream=sa)
        nb = rcs.last_grad_norm(stream=sb)
        torch.cuda.synchronize()
        _, ona = oracle.adamw_clip_step(oA[0], _host(ga), oA[1], oA[2], t, 3e-3, 0.01, 1.0)
        _, onb = oracle.adamw_clip_step(oB[0], _host(gb), oB[1], oB[2], t, 1e-3, 0.1, 2.0)
        assert abs(float(na.cpu()) - ona) <= NORM_RTOL * ona
        assert abs(float(nb.cpu()) - onb) <= NORM_RTOL * onb
    _check_state(*A, *oA, "stream A")
    _check_state(*B, *oB, "stream B")


HIP_STREAM_PER_THREAD = 2  # the hipStreamPerThread handle


@pytest.mark.parametrize("mode", ["own_streams", "per_thread_handle"])
def test_host_threads_each_on_its_own_stream(dev, mode):
    """Four host threads, each with its own stream and parameters, call the
    library at once (the ctypes calls release the GIL, so the C library sees
    concurrent calls, first-use workspace creation included); every result is
    bit-identical to the same updates run one after another. per_thread_handle:
    every thread passes hipStreamPerThread, one handle that names a different
    stream in each thread, so each thread needs a workspace of its own."""
    import threading
    sizes = [262_147, 1_000_003, 4099, 3_000_001]
    steps = 10
    init = [[workloads.custom(700 + 10 * k + j, n, 0.02 if j == 0 else 0.0, device=dev)
             for j in range(3)] for k, n in enumerate(sizes)]
    grads = [[workloads.custom(800 + 10 * k + t, n, 0.05, device=dev) for t in range(steps)]
             for k, n in enumerate(sizes)]
    ref = [[x.clone() for x in st] for st in init]
    for k in range(len(sizes)):
        for t in range(1, steps + 1):
            rcs.adamw_clip_step(ref[k][0], grads[k][t - 1], ref[k][1], ref[k][2], t, 3e-3, 0.01, 1.0)
    states = [[x.clone() for x in st] for st in init]
    streams = [torch.cuda.Stream() for _ in sizes]
    norms, errors = [None] * len(sizes), []
    torch.cuda.synchronize()
    start = threading.Barrier(len(sizes))

    def work(k):
        try:
            torch.cuda.set_device(0)
            if mode == "per_thread_handle":
                start.wait()
                w, m, v = states[k]
                for t in range(1, steps + 1):
                    rcs.adamw_clip_step(w, grads[k][t - 1], m, v, t, 3e-3, 0.01, 1.0,
                                        stream=HIP_STREAM_PER_THREAD)
                norms[k] = rcs.last_grad_norm(stream=HIP_STREAM_PER_THREAD)
                torch.cuda.synchronize()
                return
            with torch.cuda.stream(streams[k]):
                start.wait()
                w, m, v = states[k]
                for t in range(1, steps + 1):
                    rcs.adamw_clip_step(w, grads[k][t - 1], m, v, t, 3e-3, 0.01, 1.0)
                norms[k] = rcs.last_grad_norm()
            streams[k].synchronize()
        except Exception as e:  # surfaced below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(k,)) for k in range(len(sizes))]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not errors, errors
    torch.cuda.synchronize()
    for k in range(len(sizes)):
        for a, b in zip(states[k], ref[k]):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), sizes[k]
        seq = float(rcs.grad_global_norm(grads[k][-1]).cpu())
        assert float(norms[k].cpu()) == seq


@pytest.mark.parametrize("n,offset,sigma", [(1, 0, 5.0), (7, 0, 5.0), (262_147, 0, 0.01),
                                            (1_000_003, 0, 1.0), (100_001, 1, 1.0),
                                            (100_001, 2, 1.0), (7, 1, 5.0), (6, 1, 5.0),
                                            (67, 1, 5.0), (70, 1, 5.0),
                                            (8_388_611, 0, 1e-4), (8_388_613, 3, 1e-4),
                                            (12_800_000, 0, 1e-4), (124_356_866, 0, 1e-4)])
def test_grad_clip_inplace_parity(dev, n, offset, sigma):
    base = workloads.custom(600, n + offset, sigma, device=dev)
    g = base[offset:]
    og = _host(g).copy()
    rcs.grad_clip_inplace(g, 1.0)
    gn = _gpu_norm()
    rc, on = oracle.clip_grads(og, 1.0)
    assert rc == oracle.OK and abs(gn - on) <= NORM_RTOL * on
    assert max_ulp(_host(g), og) <= ULP_TOL
    if offset:
        assert (bits(_host(base[:offset])) == bits(_host(
            workloads.custom(600, n + offset, sigma, device=dev)[:offset]))).all()


def test_grad_clip_inplace_nonfinite_untouched(dev):
    g = workloads.custom(601, 10_000, 1.0, device=dev)
    g[5] = float("nan")
    before = _host(g).copy()
    rcs.grad_clip_inplace(g, 1.0)
    assert not np.isfinite(_gpu_norm())
    assert (bits(_host(g)) == bits(before)).all()


def test_gpu_path_is_deterministic(dev):
    """The reduction order depends only on n: two runs from the same state
    give the same bytes, and the same norm bit for bit, every time."""
    wl = workloads.WORKLOADS["andrea12m"]
    n = wl.n
    outs, norms = [], []
    for _ in range(2):
        w = workloads.init_params(wl, device=dev)
        m, v = workloads.zeros_like_state(n, device=dev)
        g = torch.empty(n, device=dev)
        run_norms = []
        for t in range(1, 6):
            workloads.grads(wl, t, device=dev, out=g)
            rcs.adamw_clip_step(w, g, m, v, t, wl.lr, wl.wd, wl.clip)
            run_norms.append(_gpu_norm())
        outs.append([_host(x).copy() for x in (w, m, v)])
        norms.append(run_norms)
    assert norms[0] == norms[1]
    for a, b in zip(*outs):
        assert (bits(a) == bits(b)).all()
    g = workloads.custom(700, n, 1.0, device=dev)
    vals = {float(rcs.grad_global_norm(g).cpu()) for _ in range(5)}
    assert len(vals) == 1


def test_abi_rejects_host_and_aliased_buffers(dev):
    """Host-side checks at the C boundary: pinned host memory is not device
    memory, and g aliasing w is refused, both before any launch. (Arrays
    shorter than n are refused with RCS_ESIZE when they end their allocation:
    tests/native/abi_short_buffers.c, hipMalloc'd to the exact size.)"""
    L = rcs.lib()
    n = 4096
    host = torch.zeros(n, dtype=torch.float32, pin_memory=True)
    d = [torch.zeros(n, device=dev) for _ in range(4)]
    p = [x.data_ptr() for x in d]
    stream = torch.cuda.current_stream().cuda_stream
    assert L.adamw_clip_step(host.data_ptr(), p[1], p[2], p[3], n, 1, 1e-3, 0.0, 1.0,
                             stream) == rcs.EINVAL
    assert L.adamw_clip_step(p[0], p[0], p[2], p[3], n, 1, 1e-3, 0.0, 1.0, stream) == rcs.EINVAL
    torch.cuda.synchronize()
    assert not any(x.any() for x in d)


def test_init_and_last_norm_rejections(dev):
    """rcs_init refuses a device that does not exist; last_grad_norm on a
    stream that has run nothing yet is refused rather than returning stale
    or uninitialised memory."""
    with pytest.raises(rcs.RcsError) as e:
        rcs.init(device=torch.cuda.device_count() + 7)
    assert e.value.status == rcs.EINVAL
    fresh = torch.cuda.Stream()
    rcs.init(stream=fresh)  # the workspace exists, but no norm has been computed on it
    with pytest.raises(rcs.RcsError) as e:
        rcs.last_grad_norm(stream=fresh)
    assert e.value.status == rcs.EINVAL
    g = workloads.custom(900, 1000, 1.0, device=dev)
    torch.cuda.synchronize()  # g was written on the default stream
    with torch.cuda.stream(fresh):
        rcs.grad_global_norm(g)
        got = float(rcs.last_grad_norm().cpu())
    assert abs(got - oracle.grad_norm(_host(g))) <= NORM_RTOL * got


@pytest.mark.parametrize("n", [1_000_003, 12_800_003])
def test_step_captured_in_a_graph_replays_like_eager(dev, n):
    """A caller may capture the step into its own graph once the stream's
    workspace exists (rcs_init): the capture then holds only the kernels (two
    launches at 1,000,003 elements, three at 12,800,003; no allocation, no
    memset). Each replay, with eager work and synchronizations between
    replays, gives w, m, v and the norm bit-identical to the same update run
    eagerly (t and the hyper-parameters are frozen at capture)."""
    s = torch.cuda.Stream()
    rcs.init(stream=s)
    g = workloads.custom(900, n, 0.05, device=dev)
    w0 = workloads.custom(901, n, 0.02, device=dev)
    m0 = workloads.custom(902, n, 0.01, device=dev)
    v0 = workloads.custom(903, n, 0.01, device=dev).square_()
    w, m, v = w0.clone(), m0.clone(), v0.clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        rcs.adamw_clip_step(w, g, m, v, 7, 3e-3, 0.01, 1.0)
    torch.cuda.synchronize()
    for k in range(3):
        scale = 1.0 + 0.5 * k
        w.copy_(w0 * scale)
        m.copy_(m0)
        v.copy_(v0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_norm = float(rcs.last_grad_norm(stream=s).cpu())
        we, me, ve = w0 * scale, m0.clone(), v0.clone()
        rcs.adamw_clip_step(we, g, me, ve, 7, 3e-3, 0.01, 1.0)
        eager_norm = float(rcs.last_grad_norm().cpu())
        torch.cuda.synchronize()
        for a, b in ((w, we), (m, me), (v, ve)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), (n, k)
        assert got_norm == eager_norm, (n, k, got_norm, eager_norm)
