"""Seeded synthetic workloads shared by the tests, the smoke check and bench.py.

This module holds only input recipes: sizes, parameter layouts, value
distributions and the hyper-parameters each workload is run with. It contains
none of the update's arithmetic (no norm, clip or AdamW), so both the HIP path
and the oracle can be fed from it without sharing any of the method.

Every tensor is a pure function of (base seed, workload id, stream id):
stream 0 is the parameter init, stream t >= 1 is the gradient of update t.
A run that stops at step k and resumes therefore sees exactly the gradients
of the run that never stopped.

The workloads stand in for the two models the checkpoint pages train
(ANDREA-12M, 12.8M parameters, and ANDREA-120M, whose per-layer tensors the
backprop page lists), plus a 262,144-element case small enough for the oracle
and a 2e9-element case near the int32 header limit. No dataset or trained
weight is involved; the gradients are synthetic normals.
"""
from __future__ import annotations

import dataclasses
from typing import Callable

import numpy as np
import torch

BASE_SEED = 7  # the seed of the fixed 80-update experiment in the resume lesson


def _seed(workload_id: int, stream: int, base: int = BASE_SEED) -> int:
    ss = np.random.SeedSequence([base, workload_id, stream])
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64(0x7FFF_FFFF_FFFF_FFFF))


def _gen(device: torch.device | str, workload_id: int, stream: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(workload_id, stream))
    return g


# ---- ANDREA-120M flat parameter layout in iterator order -------------------

D_MODEL, D_FF, N_LAYER, VOCAB, N_POS = 768, 3072, 12, 50257, 1024


def andrea120m_layout() -> list[tuple[str, int, str]]:
    """(name, numel, init kind) in iterator order: token and position
    embeddings, then per layer two LayerNorms (gain, bias), the four attention
    projections and the two MLP matrices, then the final LayerNorm. The output
    head is tied to the token embedding and adds no tensor."""
    segs = [("tok_emb", VOCAB * D_MODEL, "normal"), ("pos_emb", N_POS * D_MODEL, "normal")]
    for i in range(N_LAYER):
        for ln in ("ln1", "ln2"):
            segs.append((f"h{i}.{ln}.g", D_MODEL, "one"))
            segs.append((f"h{i}.{ln}.b", D_MODEL, "zero"))
        for p in ("wq", "wk", "wv", "wo"):
            segs.append((f"h{i}.{p}", D_MODEL * D_MODEL, "normal"))
        segs.append((f"h{i}.w1", D_MODEL * D_FF, "normal"))
        segs.append((f"h{i}.w2", D_FF * D_MODEL, "normal"))
    segs.append(("lnf.g", D_MODEL, "one"))
    segs.append(("lnf.b", D_MODEL, "zero"))
    return segs


ANDREA120M_N = sum(s[1] for s in andrea120m_layout())
assert ANDREA120M_N == 124_356_864


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    n: int
    steps: int
    lr: float
    wd: float
    clip: float
    grad_sigma: float
    layout: str  # "flat", "segments4", "andrea120m"
    grad_kind: str  # "normal", "outlier1pct", "outlier_every3", "stress"
    pack_at: tuple[int, ...] = ()
    description: str = ""


WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload(1, "flat262k", 262_144, 80, 3e-3, 0.01, 1.0, 1e-2, "segments4", "normal",
                 (80,), "4 contiguous 65,536-element segments; grads N(0,0.01); 80 updates"),
        Workload(2, "andrea12m", 12_800_000, 200, 3e-3, 0.01, 1.0, 1e-3, "flat", "outlier1pct",
                 (100, 200), "12.8M flat; grads N(0,1e-3), 1% of elements x100 each step"),
        Workload(6, "andrea12m_b", 12_800_000, 200, 3e-3, 0.01, 1.0, 1e-4, "flat",
                 "outlier_every3", (100, 200),
                 "12.8M flat; grads N(0,1e-4), 1% x100 only on steps t%3==0 (clip fires "
                 "on those steps only)"),
        Workload(3, "andrea120m", ANDREA120M_N, 100, 3e-3, 0.01, 1.0, 1e-4, "andrea120m",
                 "normal", (), "ANDREA-120M layout, 124,356,864 params (matrices N(0,0.02), "
                 "LayerNorm gains 1 and biases 0); grads N(0,1e-4)"),
        Workload(4, "andrea120m_stress", ANDREA120M_N, 200, 3e-3, 0.01, 1.0, 1.0, "andrea120m",
                 "stress", (100,), "ANDREA-120M layout; grads N(0,1), 5% exact zeros, 0.1% "
                 "+-U[0.5,2]e-38 (subnormal and near FLT_MIN)"),
        Workload(5, "flat2e9", 2_000_000_000, 10, 1e-4, 0.01, 1.0, 1e-4, "flat", "normal", (10,),
                 "2e9 flat params near the int32 header limit; grads N(0,1e-4)"),
    ]
}


def init_params(wl: Workload, device="cpu", n: int | None = None) -> torch.Tensor:
    """Parameter init (stream 0): N(0, 0.02) for matrices and embeddings,
    LayerNorm gain 1 and bias 0. ``n`` truncates to a prefix (small tests)."""
    n_full = wl.n
    n = n_full if n is None else n
    w = torch.randn(n, generator=_gen(device, wl.wid, 0), device=device,
                    dtype=torch.float32).mul_(0.02)
    if wl.layout == "andrea120m":
        off = 0
        for _, numel, kind in andrea120m_layout():
            if off >= n:
                break
            hi = min(off + numel, n)
            if kind == "one":
                w[off:hi] = 1.0
            elif kind == "zero":
                w[off:hi] = 0.0
            off += numel
    return w


def grads(wl: Workload, t: int, device="cpu", n: int | None = None,
          out: torch.Tensor | None = None) -> torch.Tensor:
    """Gradient of update t (t >= 1), a pure function of (workload, t)."""
    if t < 1:
        raise ValueError("gradient streams start at t = 1")
    n = wl.n if n is None else n
    gen = _gen(device, wl.wid, t)
    g = out if out is not None else torch.empty(n, device=device, dtype=torch.float32)
    g.normal_(0.0, 1.0, generator=gen).mul_(wl.grad_sigma)
    if wl.grad_kind in ("outlier1pct", "outlier_every3"):
        if wl.grad_kind == "outlier1pct" or t % 3 == 0:
            sel = torch.rand(n, generator=gen, device=device) < 0.01
            g[sel] *= 100.0
    elif wl.grad_kind == "stress":
        u = torch.rand(n, generator=gen, device=device)
        g[u < 0.05] = 0.0
        tiny = (u >= 0.05) & (u < 0.051)
        k = int(tiny.sum().item())
        mag = torch.empty(k, device=device, dtype=torch.float32).uniform_(0.5, 2.0,
                                                                          generator=gen)
        sign = torch.where(torch.rand(k, generator=gen, device=device) < 0.5, -1.0, 1.0)
        g[tiny] = (mag * 1e-38 * sign).to(torch.float32)
    elif wl.grad_kind != "normal":
        raise ValueError(wl.grad_kind)
    return g


def zeros_like_state(n: int, device="cpu") -> tuple[torch.Tensor, torch.Tensor]:
    return (torch.zeros(n, device=device, dtype=torch.float32),
            torch.zeros(n, device=device, dtype=torch.float32))


def custom(wid: int, n: int, sigma: float, device="cpu", stream: int = 1) -> torch.Tensor:
    """A free-standing N(0, sigma) vector for edge-case tests."""
    return torch.randn(n, generator=_gen(device, wid, stream), device=device,
                       dtype=torch.float32).mul_(sigma)


GradFn = Callable[[int], torch.Tensor]
