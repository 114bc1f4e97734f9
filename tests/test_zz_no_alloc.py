"""adamw_clip_step_noalloc through the C ABI against adamw_clip_step.

The no-allocation entry point keeps the norm pass's partials and the clip
record in the library's static device array instead of the per-stream
workspace; its kernels and arithmetic are those of adamw_clip_step, so w, m, v
and the norm must come out bit-identical. Two calls in a row, the second with
a smaller input (the array keeps the first call's contents), in both launch
forms (three kernels above 8,388,608 elements, two below), then host-side
rejections that launch nothing.
"""
import ctypes

import numpy as np
import pytest
import torch

import resumable_checkpoint_state_amd as rcs
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rcs.lib()
    torch.cuda.set_device(0)
    return torch.device("cuda:0")


def _state(n, seed, dev):
    w = workloads.custom(seed, n, 0.02, device=dev)
    g = workloads.custom(seed + 1, n, 0.05, device=dev)
    m = workloads.custom(seed + 2, n, 0.01, device=dev)
    v = workloads.custom(seed + 3, n, 0.01, device=dev).square_()
    return w, g, m, v


def test_noalloc_matches_the_workspace_entry_point(dev):
    L = rcs.lib()
    stream = torch.cuda.current_stream().cuda_stream
    for call, (n, t) in enumerate([(12_800_003, 5), (1_000_003, 6)]):
        w, g, m, v = _state(n, 1000 + 10 * call, dev)
        we, me, ve = w.clone(), m.clone(), v.clone()
        norm_dev = torch.full((1,), -1.0, dtype=torch.float64, device=dev)
        norm_host = torch.full((1,), -1.0, dtype=torch.float64, pin_memory=True)
        torch.cuda.synchronize()
        print(f"no-alloc call {call}: n={n} t={t}", flush=True)
        rc = L.adamw_clip_step_noalloc(w.data_ptr(), g.data_ptr(), m.data_ptr(), v.data_ptr(), n,
                                       t, 3e-3, 0.01, 1.0, norm_dev.data_ptr(), stream)
        assert rc == rcs.OK, rcs.strerror(rc)
        # the same update again into fresh copies, norm into pinned host memory
        w2, m2, v2 = we.clone(), me.clone(), ve.clone()
        rc = L.adamw_clip_step_noalloc(w2.data_ptr(), g.data_ptr(), m2.data_ptr(),
                                       v2.data_ptr(), n, t, 3e-3, 0.01, 1.0,
                                       norm_host.data_ptr(), stream)
        assert rc == rcs.OK, rcs.strerror(rc)
        rc = L.adamw_clip_step(we.data_ptr(), g.data_ptr(), me.data_ptr(), ve.data_ptr(), n, t,
                               3e-3, 0.01, 1.0, stream)
        assert rc == rcs.OK, rcs.strerror(rc)
        ref_norm = float(rcs.last_grad_norm().cpu())
        torch.cuda.synchronize()
        assert ref_norm > 1.0  # the clip fires
        assert np.float64(norm_dev.item()).tobytes() == np.float64(ref_norm).tobytes()
        assert np.float64(norm_host.item()).tobytes() == np.float64(ref_norm).tobytes()
        for a, a2, b in ((w, w2, we), (m, m2, me), (v, v2, ve)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), (n, call)
            assert torch.equal(a2.view(torch.int32), b.view(torch.int32)), (n, call)


def test_noalloc_without_a_norm_destination_and_on_views(dev):
    """norm_out = NULL; arrays at another 16-byte phase (the mixed kernels)."""
    L = rcs.lib()
    stream = torch.cuda.current_stream().cuda_stream
    n = 70_001
    W, G, M, V = (torch.zeros(n + 3, device=dev) for _ in range(4))
    w, g, m, v = W[1:n + 1], G[3:], M[1:n + 1], V[2:n + 2]
    w.copy_(workloads.custom(1100, n, 0.02, device=dev))
    g.copy_(workloads.custom(1101, n, 0.05, device=dev))
    we, me, ve = w.clone(), m.clone(), v.clone()
    rc = L.adamw_clip_step_noalloc(w.data_ptr(), g.data_ptr(), m.data_ptr(), v.data_ptr(), n, 2,
                                   1e-3, 0.1, 0.5, None, stream)
    assert rc == rcs.OK
    rcs.adamw_clip_step(we, g, me, ve, 2, 1e-3, 0.1, 0.5)
    torch.cuda.synchronize()
    for a, b in ((w, we), (m, me), (v, ve)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_noalloc_rejections_launch_nothing(dev):
    L = rcs.lib()
    stream = torch.cuda.current_stream().cuda_stream
    n = 4096
    w, g, m, v = (torch.zeros(n, device=dev) for _ in range(4))
    p = [x.data_ptr() for x in (w, g, m, v)]
    # n beyond the header's limit, t < 1, a bad clip
    assert L.adamw_clip_step_noalloc(*p, rcs.MAX_N + 1, 1, 1e-3, 0.0, 1.0, None,
                                     stream) == rcs.EINVAL
    assert L.adamw_clip_step_noalloc(*p, n, 0, 1e-3, 0.0, 1.0, None, stream) == rcs.EINVAL
    assert L.adamw_clip_step_noalloc(*p, n, 1, 1e-3, 0.0, 0.0, None, stream) == rcs.EINVAL
    # a norm destination in pageable host memory is refused before any launch
    pageable = (ctypes.c_double * 1)(-1.0)
    assert L.adamw_clip_step_noalloc(*p, n, 1, 1e-3, 0.0, 1.0, ctypes.addressof(pageable),
                                     stream) == rcs.EINVAL
    torch.cuda.synchronize()
    assert not w.any() and not m.any() and not v.any()
