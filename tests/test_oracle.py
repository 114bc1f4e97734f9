"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: the values
the resume lesson prints for its one-dimensional example, closed forms,
exact rational arithmetic, PyTorch's own AdamW and clip routines in float64,
and the byte layout written out with Python's struct module.
"""
import json
import math
import os
import struct
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f32bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


# ---------------------------------------------------------------- worked example

def test_subnormals_kept_in_process():
    assert oracle.subnormals_kept()


def _f64(*xs):
    return np.array(xs, dtype=np.float64)


def test_worked_example_float64_definition():
    """The update's definition in float64 on the one-dimensional example:
    the moments, their bias-corrected values, the decayed weight and the
    weight after the step printed on the page."""
    ex = _golden("worked_example_1d.json")
    inp, s1 = ex["inputs"], ex["step1"]
    w, g, m, v = _f64(inp["theta0"]), _f64(inp["grads"][0]), _f64(0), _f64(0)
    rc, norm = oracle.adamw_clip_step_f64(w, g, m, v, 1, inp["lr"], inp["wd"], inp["clip"])
    assert rc == oracle.OK and norm == abs(inp["grads"][0])  # below the threshold: no clip
    assert abs(w[0] - s1["theta"]) < s1["theta_abs_tol"]
    # (1 - beta) is formed in float64, a few ulps off the decimal figures
    assert m[0] == pytest.approx(s1["m"], rel=4e-15)
    assert v[0] == pytest.approx(s1["v"], rel=4e-15)
    assert m[0] / (1 - 0.9) == pytest.approx(s1["m_hat"], rel=1e-14)
    assert v[0] / (1 - 0.999) == pytest.approx(s1["v_hat"], rel=1e-12)
    # the decayed weight: the step is lr * m_hat / sqrt(v_hat) = 0.1 off it
    assert inp["theta0"] * (1 - inp["lr"] * inp["wd"]) == pytest.approx(s1["decayed_theta"])
    assert s1["decayed_theta"] - w[0] == pytest.approx(s1["adaptive_step"], abs=1e-7)


def test_float64_definition_clips_the_whole_vector():
    """g = (3, 4) has norm 5; with clip 1 the whole vector is scaled by 1/5
    (direction kept), so at t = 1 m = 0.1 * (0.6, 0.8) and v = 0.001 * g'^2."""
    w, g, m, v = _f64(1.0, -1.0), _f64(3.0, 4.0), _f64(0, 0), _f64(0, 0)
    rc, norm = oracle.adamw_clip_step_f64(w, g, m, v, 1, 0.01, 0.0, 1.0)
    assert rc == oracle.OK and norm == 5.0
    assert m == pytest.approx([0.06, 0.08], rel=1e-14)
    assert v == pytest.approx([0.001 * 0.36, 0.001 * 0.64], rel=1e-13)
    # m_hat = g', v_hat = g'^2: each weight moves by lr * |g'| / (|g'| + eps) ~ lr
    assert w == pytest.approx([1.0 - 0.01, -1.0 - 0.01], abs=1e-9)
    g[1] = np.inf
    assert oracle.adamw_clip_step_f64(w, g, m, v, 2, 0.01, 0.0, 1.0)[0] == oracle.SKIPPED


def test_float64_definition_resume_needs_the_whole_state():
    """Six updates of a seven-element vector straight through equal three, a
    round trip of (w, m, v) through their bytes, and three more from t = 4;
    restarting with the weights only (m = v = 0, t from 1) does not."""
    rng = np.random.default_rng(11)
    w0 = rng.standard_normal(7)
    gs = [rng.standard_normal(7) * 0.3 for _ in range(6)]
    hp = (0.05, 0.01, 1.0)
    w, m, v = w0.copy(), np.zeros(7), np.zeros(7)
    for t, g in enumerate(gs, start=1):
        oracle.adamw_clip_step_f64(w, g, m, v, t, *hp)
    w2, m2, v2 = w0.copy(), np.zeros(7), np.zeros(7)
    for t, g in enumerate(gs[:3], start=1):
        oracle.adamw_clip_step_f64(w2, g, m2, v2, t, *hp)
    blob = w2.tobytes() + m2.tobytes() + v2.tobytes()
    w3, m3, v3 = (np.frombuffer(blob[k * 56:(k + 1) * 56], dtype=np.float64).copy()
                  for k in range(3))
    for t, g in enumerate(gs[3:], start=4):
        oracle.adamw_clip_step_f64(w3, g, m3, v3, t, *hp)
    assert w3.tobytes() == w.tobytes() and m3.tobytes() == m.tobytes()
    assert v3.tobytes() == v.tobytes()
    w4, m4, v4 = w2.copy(), np.zeros(7), np.zeros(7)
    for t, g in enumerate(gs[3:], start=1):
        oracle.adamw_clip_step_f64(w4, g, m4, v4, t, *hp)
    assert np.abs(w4 - w).max() > 1e-3


def _vec(x):
    return np.array([x], dtype=np.float32)


def test_worked_example_float32_vector_step():
    """The float32 sequence on the same example lands on the page's values
    rounded to float32."""
    ex = _golden("worked_example_1d.json")
    inp, s1 = ex["inputs"], ex["step1"]
    w, g, m, v = _vec(inp["theta0"]), _vec(inp["grads"][0]), _vec(0), _vec(0)
    rc, norm = oracle.adamw_clip_step(w, g, m, v, 1, inp["lr"], inp["wd"], inp["clip"])
    assert rc == oracle.OK and norm == 0.5
    assert f32bits(m[0]) == f32bits(np.float32(s1["m"]))
    assert f32bits(v[0]) == f32bits(np.float32(s1["v"]))
    assert f32bits(w[0]) == f32bits(np.float32(s1["theta"]))
    bc1, bc2, decay = oracle.scalars(1, inp["lr"], inp["wd"])
    assert np.float32(m[0] / bc1) == np.float32(s1["m_hat"])
    assert np.float32(v[0] / bc2) == np.float32(s1["v_hat"])
    assert np.float32(np.float32(inp["theta0"]) * decay) == np.float32(s1["decayed_theta"])


def test_worked_example_float32_three_steps_and_resume():
    ex = _golden("worked_example_1d.json")
    inp = ex["inputs"]
    hp = (inp["lr"], inp["wd"], inp["clip"])
    # straight
    w, m, v = _vec(inp["theta0"]), _vec(0), _vec(0)
    for t, g in enumerate(inp["grads"], start=1):
        assert oracle.adamw_clip_step(w, _vec(g), m, v, t, *hp)[0] == oracle.OK
    # two steps, pack, unpack into fresh arrays, one more step
    w2, m2, v2 = _vec(inp["theta0"]), _vec(0), _vec(0)
    for t, g in enumerate(inp["grads"][:2], start=1):
        oracle.adamw_clip_step(w2, _vec(g), m2, v2, t, *hp)
    rc, buf = oracle.ckpt_pack(2, w2, m2, v2)
    assert rc == oracle.OK
    w3, m3, v3 = _vec(9), _vec(9), _vec(9)
    rc, step = oracle.ckpt_unpack(buf, w3, m3, v3)
    assert rc == oracle.OK and step == 2
    oracle.adamw_clip_step(w3, _vec(inp["grads"][2]), m3, v3, step + 1, *hp)
    assert f32bits(w3) == f32bits(w) and f32bits(m3) == f32bits(m) and f32bits(v3) == f32bits(v)
    # the float32 sequence tracks the float64 definition within a few float32 ulps
    w64, m64, v64 = _f64(inp["theta0"]), _f64(0), _f64(0)
    for t, g in enumerate(inp["grads"], start=1):
        oracle.adamw_clip_step_f64(w64, _f64(g), m64, v64, t, *hp)
    assert abs(float(w[0]) - w64[0]) <= 4 * np.spacing(np.float32(w64[0]))
    assert abs(float(m[0]) - m64[0]) <= 4 * np.spacing(np.float32(m64[0]))
    assert abs(float(v[0]) - v64[0]) <= 4 * np.spacing(np.float32(v64[0]))
    # weights-only resume (m = v = 0, t restarts) diverges
    ww, mm, vv = w2.copy(), _vec(0), _vec(0)
    oracle.adamw_clip_step(ww, _vec(inp["grads"][2]), mm, vv, 1, *hp)
    assert abs(float(ww[0]) - float(w[0])) > ex["resume"]["weights_only_resume_min_abs_diff"]


# ---------------------------------------------------------------- norm

def _exact_norm(g):
    s = sum((Fraction(float(x)) ** 2 for x in g), Fraction(0))
    getcontext().prec = 60
    return Fraction(s), Decimal(s.numerator) / Decimal(s.denominator)


def test_norm_against_exact_rational_sum():
    rng = np.random.default_rng(11)
    for n, scale in [(1, 1.0), (7, 1e-3), (1000, 1.0), (4099, 1e-20), (10000, 1e15)]:
        g = (rng.standard_normal(n) * scale).astype(np.float32)
        g[::97] *= np.float32(1e3)  # spread exponents
        s_exact, s_dec = _exact_norm(g)
        s = oracle.sumsq(g)
        assert abs(Fraction(s) - s_exact) <= s_exact * Fraction(1, 2**52), (n, scale)
        norm_exact = float(s_dec.sqrt())
        assert abs(oracle.grad_norm(g) - norm_exact) <= 2.3e-16 * norm_exact


def test_norm_streamed_chunks_equal_one_pass():
    g = np.random.default_rng(3).standard_normal(50_001).astype(np.float32)
    acc = oracle.NormAccumulator()
    for lo in range(0, g.size, 7_777):
        acc.add(g[lo:lo + 7_777])
    assert acc.norm() == oracle.grad_norm(g)


def test_norm_powers_of_two_exact():
    n = 1 << 18
    assert oracle.grad_norm(np.full(n, 2.0 ** -6, np.float32)) == 8.0
    assert oracle.clip_scale(8.0, 1.0) == np.float32(0.125)
    assert oracle.grad_norm(np.full(n, 2.0 ** -10, np.float32)) == 0.5
    assert oracle.clip_scale(0.5, 1.0) == np.float32(1.0)
    one = np.zeros(n, np.float32)
    one[12345] = -3.25
    assert oracle.grad_norm(one) == 3.25
    assert oracle.grad_norm(np.zeros(n, np.float32)) == 0.0


def test_norm_matches_torch_clip_grad_norm_total():
    g = (np.random.default_rng(5).standard_normal(100_000) * 0.01).astype(np.float32)
    p = torch.nn.Parameter(torch.zeros(g.size, dtype=torch.float64))
    p.grad = torch.from_numpy(g.astype(np.float64))
    total = float(torch.nn.utils.clip_grad_norm_([p], max_norm=1e30))
    assert oracle.grad_norm(g) == pytest.approx(total, rel=1e-13)


def test_norm_nonfinite_skips_update():
    w = np.ones(8, np.float32)
    m = np.full(8, 0.5, np.float32)
    v = np.full(8, 0.25, np.float32)
    for bad in (np.inf, -np.inf, np.nan):
        g = np.ones(8, np.float32)
        g[3] = bad
        w0, m0, v0 = w.copy(), m.copy(), v.copy()
        rc, norm = oracle.adamw_clip_step(w, g, m, v, 5, 1e-3, 0.01, 1.0)
        assert rc == oracle.SKIPPED and not math.isfinite(norm)
        assert (norm == math.inf) if not np.isnan(bad) else math.isnan(norm)
        assert (f32bits(w) == f32bits(w0)).all() and (f32bits(m) == f32bits(m0)).all()
        assert (f32bits(v) == f32bits(v0)).all()
    # huge finite values overflow the float32 square but not the float64 sum
    g = np.full(8, 3e38, np.float32)
    rc, norm = oracle.adamw_clip_step(w, g, m, v, 5, 1e-3, 0.01, 1.0)
    assert rc == oracle.OK and norm == pytest.approx(3e38 * math.sqrt(8), rel=1e-7)


# ---------------------------------------------------------------- clip

def test_clip_invariants_through_update():
    """At t=1 with m=v=0 and wd=0 the new m is 0.1*g', so the clipped
    gradient is visible: ||g'|| <= c, signs kept, g'/g constant."""
    rng = np.random.default_rng(1)
    for sigma, clip in [(0.01, 1.0), (1.0, 1.0), (1e-4, 1.0), (3.0, 0.25)]:
        n = 40_000
        g = (rng.standard_normal(n) * sigma).astype(np.float32)
        w, m, v = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32)
        rc, norm = oracle.adamw_clip_step(w, g, m, v, 1, 1e-3, 0.0, clip)
        assert rc == oracle.OK
        gp = m.astype(np.float64) / np.float64(np.float32(0.1))
        gp_norm = np.sqrt(np.sum(gp * gp))
        if norm > clip:
            assert gp_norm <= clip * (1 + 8 * 2.0 ** -24)
            assert gp_norm == pytest.approx(clip, rel=1e-6)
        else:
            # below the threshold the gradient is left alone: m = 0.1f * g exactly
            assert (f32bits(m) == f32bits(np.float32(0.1) * g)).all()
        nz = g != 0
        assert (np.sign(m[nz]) == np.sign(g[nz])).all()
        ratio = gp[nz] / g[nz].astype(np.float64)
        assert ratio.max() / ratio.min() - 1 < 1e-6


def test_clip_scale_properties():
    for norm in [1.0000001, 1.5, 7.0, 123.456, 1e30, 10863.0]:
        s = oracle.clip_scale(norm, 1.0)
        assert 0 < s < 1
        assert float(s) * norm <= 1.0 * (1 + 2.0 ** -23)
    assert oracle.clip_scale(1.0, 1.0) == 1.0  # strict '>' threshold
    assert oracle.clip_scale(0.0, 1.0) == 1.0
    assert oracle.clip_scale(5.0, float("inf")) == 1.0


# ---------------------------------------------------------------- AdamW vs library

@pytest.mark.parametrize("sigma,clip", [(0.01, 1e9), (0.01, 1.0), (1.0, 1.0)])
def test_trajectory_matches_torch_adamw_float64(sigma, clip):
    """PyTorch's AdamW and clip_grad_norm_ in float64 follow the same maths
    (their clip adds 1e-6 to the norm, a relative change far below the
    tolerance after Adam's normalisation)."""
    n, steps, lr, wd = 5000, 30, 1e-2, 0.1
    rng = np.random.default_rng(21)
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    p = torch.nn.Parameter(torch.from_numpy(w.astype(np.float64)))
    opt = torch.optim.AdamW([p], lr=lr, betas=(0.9, 0.999), eps=1e-8, weight_decay=wd)
    for t in range(1, steps + 1):
        g = (rng.standard_normal(n) * sigma).astype(np.float32)
        oracle.adamw_clip_step(w, g, m, v, t, lr, wd, clip)
        p.grad = torch.from_numpy(g.astype(np.float64))
        torch.nn.utils.clip_grad_norm_([p], max_norm=clip)
        opt.step()
    ref = p.detach().numpy()
    st = opt.state[p]
    assert np.abs(w - ref).max() <= 2e-6 * np.abs(ref).max()
    assert np.allclose(m, st["exp_avg"].numpy(), rtol=2e-5, atol=1e-7 * sigma)
    assert np.allclose(v, st["exp_avg_sq"].numpy(), rtol=2e-5, atol=1e-9 * sigma * sigma)


def test_special_case_lr_zero_leaves_w_bit_identical():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal(1000) * 0.02).astype(np.float32)
    w[0], w[1] = -0.0, 0.0
    w0 = w.copy()
    m, v = np.zeros_like(w), np.zeros_like(w)
    for t in range(1, 4):
        g = rng.standard_normal(1000).astype(np.float32)
        oracle.adamw_clip_step(w, g, m, v, t, 0.0, 0.01, 1.0)
    # -0.0 minus a +-0 step may come out +0.0 (IEEE), equal in value
    assert (w == w0).all()
    nz = w0 != 0
    assert (f32bits(w[nz]) == f32bits(w0[nz])).all()


def test_special_case_zero_grad_is_pure_decay():
    rng = np.random.default_rng(4)
    w = (rng.standard_normal(1000) * 0.02).astype(np.float32)
    m, v = np.zeros_like(w), np.zeros_like(w)
    g = np.zeros_like(w)
    _, _, decay = oracle.scalars(1, 3e-3, 0.01)
    assert decay == np.float32(1 - 3e-5)
    expect = w.copy()
    for t in range(1, 6):
        oracle.adamw_clip_step(w, g, m, v, t, 3e-3, 0.01, 1.0)
        expect = (expect * decay).astype(np.float32)
    assert (f32bits(w) == f32bits(expect)).all()
    assert not m.any() and not v.any()


def test_special_case_constant_grad_closed_form():
    """wd = 0 and constant g: in exact arithmetic m_hat = g and v_hat = g^2 at
    every t, so w_t = w_0 - t*lr*g/(|g|+eps)."""
    n, steps, lr = 64, 50, 1e-3
    for gval in [0.3, -2.0, 1e-8, -1e-8]:
        w = np.linspace(-1, 1, n).astype(np.float32)
        w0 = w.astype(np.float64)
        m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
        g = np.full(n, gval, np.float32)
        for t in range(1, steps + 1):
            oracle.adamw_clip_step(w, g, m, v, t, lr, 0.0, float("inf"))
        g64 = float(np.float32(gval))
        expect = w0 - steps * lr * g64 / (abs(g64) + 1e-8)
        # one float32 rounding of w per step plus a relative 1e-5 on each step size
        tol = steps * (float(np.spacing(np.float32(1.1))) + lr * 1e-5)
        assert np.abs(w - expect).max() < tol, gval


def test_scalars_bias_correction_and_decay():
    for t in [1, 2, 10, 100, 1000, 16000, 2**31 - 1]:
        bc1, bc2, _ = oracle.scalars(t, 3e-3, 0.01)
        assert bc1 == np.float32(1 - 0.9 ** t)
        assert bc2 == np.float32(1 - 0.999 ** t)
    _, _, d = oracle.scalars(1, 0.1, 0.01)
    assert d == np.float32(1 - np.float64(np.float32(0.1)) * np.float64(np.float32(0.01)))


def test_invalid_arguments_rejected():
    a = np.zeros(4, np.float32)
    assert oracle.adamw_clip_step(a, a.copy(), a.copy(), a.copy(), 0, 1e-3, 0.0, 1.0)[0] \
        == oracle.EINVAL
    assert oracle.adamw_clip_step(a, a.copy(), a.copy(), a.copy(), 1, float("nan"), 0.0,
                                  1.0)[0] == oracle.EINVAL
    assert oracle.adamw_clip_step(a, a.copy(), a.copy(), a.copy(), 1, 1e-3, 0.0, 0.0)[0] \
        == oracle.EINVAL
    assert oracle.adamw_clip_step(a, a.copy(), a.copy(), a.copy(), 1, 1e-3, 0.0, -1.0)[0] \
        == oracle.EINVAL


# ---------------------------------------------------------------- state layout

def test_ckpt_bytes_closed_form_and_printed_sizes():
    gold = _golden("checkpoint_sizes.json")
    for n in [1, 4, 262_144, 12_800_000, 124_356_864, 2_000_000_000, 2**31 - 1]:
        assert oracle.ckpt_bytes(n) == 8 + 12 * n
    for bad in [0, -1, 2**31, 2**40]:
        assert oracle.ckpt_bytes(bad) == -1
    a12 = gold["printed"][0]
    nb = oracle.ckpt_bytes(a12["n_params"])
    assert nb == 153_600_008
    assert round(nb / 1e6) == a12["MB_1e6_rounded"]
    # 146.48 MiB: the page's "147 MB rounded" is that figure rounded up
    assert math.ceil(nb / 2**20) == a12["MiB_rounded"]
    a120 = gold["printed"][1]
    assert oracle.ckpt_bytes(a120["n_params_approx"]) / 1e9 == pytest.approx(
        a120["GB_1e9_approx"], abs=0.005)
    assert oracle.ckpt_bytes(124_356_864) == 1_492_282_376


def test_pack_layout_matches_struct_and_numpy():
    rng = np.random.default_rng(8)
    n = 1001
    w = rng.standard_normal(n).astype(np.float32)
    m = rng.standard_normal(n).astype(np.float32)
    v = rng.random(n).astype(np.float32)
    w[:4] = [np.float32(-0.0), np.float32(1e-45), np.float32(np.inf), np.float32(np.nan)]
    rc, buf = oracle.ckpt_pack(123456, w, m, v)
    assert rc == oracle.OK and buf.size == 8 + 12 * n
    expect = struct.pack("<ii", 123456, n) + w.astype("<f4").tobytes() + \
        m.astype("<f4").tobytes() + v.astype("<f4").tobytes()
    assert buf.tobytes() == expect
    assert oracle.ckpt_header(buf) == (oracle.OK, 123456, n)
    w2, m2, v2 = (np.empty(n, np.float32) for _ in range(3))
    rc, step = oracle.ckpt_unpack(buf, w2, m2, v2)
    assert rc == oracle.OK and step == 123456
    for a, b in [(w, w2), (m, m2), (v, v2)]:
        assert (f32bits(a) == f32bits(b)).all()


def test_pack_file_name_pattern():
    assert "step_%06d.bin" % 112700 == "step_112700.bin"
    assert "step_%06d.bin" % 80 == "step_000080.bin"


@pytest.mark.parametrize("case", ["truncated", "extended", "n_zero", "n_negative", "n_mismatch",
                                  "step_negative", "short_header"])
def test_unpack_rejects_bad_buffers_and_leaves_outputs(case):
    n = 16
    w = np.arange(n, dtype=np.float32)
    rc, buf = oracle.ckpt_pack(7, w, w + 1, w + 2)
    assert rc == oracle.OK
    want = oracle.EHEADER
    if case == "truncated":
        buf, want = buf[:-1].copy(), oracle.ESIZE
    elif case == "extended":
        buf, want = np.concatenate([buf, np.zeros(1, np.uint8)]), oracle.ESIZE
    elif case == "n_zero":
        buf[4:8] = np.frombuffer(struct.pack("<i", 0), np.uint8)
    elif case == "n_negative":
        buf[4:8] = np.frombuffer(struct.pack("<i", -16), np.uint8)
    elif case == "n_mismatch":
        buf[4:8] = np.frombuffer(struct.pack("<i", 15), np.uint8)
    elif case == "step_negative":
        buf[0:4] = np.frombuffer(struct.pack("<i", -1), np.uint8)
    elif case == "short_header":
        buf, want = buf[:7].copy(), oracle.ESIZE
    outs = [np.full(n, 42.0, np.float32) for _ in range(3)]
    rc, _ = oracle.ckpt_unpack(buf, *outs)
    assert rc == want
    assert all((o == 42.0).all() for o in outs)


def test_pack_rejects_wrong_buffer_size():
    w = np.zeros(10, np.float32)
    rc, _ = oracle.ckpt_pack(1, w, w, w, buf=np.zeros(8 + 12 * 10 - 1, np.uint8))
    assert rc == oracle.ESIZE
    rc, _ = oracle.ckpt_pack(-1, w, w, w)
    assert rc == oracle.EINVAL


def test_straight_equals_pack_resume_small_trajectory():
    import workloads
    wl = workloads.WORKLOADS["flat262k"]
    n = 20_000
    w0 = workloads.init_params(wl, n=n).numpy()
    grads = [workloads.grads(wl, t, n=n).numpy() for t in range(1, 11)]
    hp = (wl.lr, wl.wd, wl.clip)
    w, m, v = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in range(1, 11):
        oracle.adamw_clip_step(w, grads[t - 1], m, v, t, *hp)
    w2, m2, v2 = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in range(1, 6):
        oracle.adamw_clip_step(w2, grads[t - 1], m2, v2, t, *hp)
    _, buf = oracle.ckpt_pack(5, w2, m2, v2)
    w3, m3, v3 = (np.empty(n, np.float32) for _ in range(3))
    _, step = oracle.ckpt_unpack(buf, w3, m3, v3)
    for t in range(step + 1, 11):
        oracle.adamw_clip_step(w3, grads[t - 1], m3, v3, t, *hp)
    assert oracle.ckpt_pack(10, w, m, v)[1].tobytes() == \
        oracle.ckpt_pack(10, w3, m3, v3)[1].tobytes()


# ---------------------------------------------------------------- micro-batch accumulation

def test_scale_grads_averages_accumulated_microbatches():
    """Backward passes add into one buffer, then the sum is multiplied by
    1/n_micro: two identical micro-batches average back to the gradient
    exactly (g + g = 2g and 2g * 0.5 = g are exact); three come back within
    one float32 rounding of each step."""
    g = (np.random.default_rng(31).standard_normal(10_000) * 0.01).astype(np.float32)
    two = (g + g).astype(np.float32)
    oracle.scale_grads(two, 0.5)
    assert (f32bits(two) == f32bits(g)).all()
    three = ((g + g) + g).astype(np.float32)
    oracle.scale_grads(three, float(np.float32(1) / np.float32(3)))
    assert np.abs(three.astype(np.float64) - g) .max() <= 3 * np.spacing(np.abs(g)).max()
    # the accumulated step equals the plain step on the averaged gradient
    w1, m1, v1 = np.full(g.size, 0.5, np.float32), np.zeros_like(g), np.zeros_like(g)
    w2, m2, v2 = w1.copy(), m1.copy(), v1.copy()
    oracle.adamw_clip_step_accum(w1, (g + g).astype(np.float32), m1, v1, 1, 3e-3, 0.01, 1.0, 0.5)
    oracle.adamw_clip_step(w2, g, m2, v2, 1, 3e-3, 0.01, 1.0)
    assert (f32bits(w1) == f32bits(w2)).all() and (f32bits(m1) == f32bits(m2)).all()


# ---------------------------------------------------------------- the clip on its own

def test_clip_grads_matches_torch_and_the_update_path():
    rng = np.random.default_rng(41)
    for sigma, clip in [(0.01, 1.0), (1.0, 1.0), (3.0, 0.25), (1e-4, 1.0)]:
        g = (rng.standard_normal(30_000) * sigma).astype(np.float32)
        g0 = g.copy()
        rc, norm = oracle.clip_grads(g, clip)
        assert rc == oracle.OK
        # PyTorch's clip in float64 (its factor has +1e-6 in the denominator)
        p = torch.nn.Parameter(torch.zeros(g.size, dtype=torch.float64))
        p.grad = torch.from_numpy(g0.astype(np.float64))
        total = float(torch.nn.utils.clip_grad_norm_([p], max_norm=clip))
        assert norm == pytest.approx(total, rel=1e-13)
        assert np.allclose(g, p.grad.numpy(), rtol=2e-6 + 2e-6 / norm, atol=0)
        if norm <= clip:
            assert (f32bits(g) == f32bits(g0)).all()
        else:
            assert np.sqrt(np.sum(g.astype(np.float64) ** 2)) <= clip * (1 + 8 * 2.0 ** -24)
        # the update applies the same clipped gradient: at t = 1 with m = 0, m = 0.1f * g'
        w, m, v = np.zeros_like(g0), np.zeros_like(g0), np.zeros_like(g0)
        oracle.adamw_clip_step(w, g0, m, v, 1, 1e-3, 0.0, clip)
        assert (f32bits(m) == f32bits(np.float32(0.1) * g)).all()


def test_clip_grads_nonfinite_leaves_gradient():
    g = np.ones(100, np.float32)
    g[7] = np.inf
    g0 = g.copy()
    rc, norm = oracle.clip_grads(g, 1.0)
    assert rc == oracle.SKIPPED and norm == np.inf
    assert (f32bits(g) == f32bits(g0)).all()
