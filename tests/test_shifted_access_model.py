"""A lane-by-lane model, on the CPU, of how the update and snapshot kernels
read and write an array that lies q = 1-3 floats off the 16-byte phase of
the body (csrc/rcs.hip: ld_shifted / st_shifted and the head/tail split of
update_body). One wave is 64 lanes; lane i of the body owns elements
xb[4i .. 4i+3]; it loads the aligned vector holding its first element, takes
the rest from the next lane, and stores the aligned vector holding its first
element from the previous lane's last elements and its own first ones; lane
0, lane 63 and the body's first and last vectors move their missing elements
one by one.

The model checks what the kernels rely on, for every phase, heads of 0-7 and
60-63 elements and bodies of 4 to 12,800 elements:
- every access stays inside the array (no read or write outside
  [0, head + body));
- every lane sees exactly its own four elements;
- every body element is written exactly once, with its own lane's value;
- run with waves in random order against memory that each wave's stores
  change at once, every element a lane uses is still the value from before
  any store (a wave reads only what it or the next lane of the same wave
  loaded before that wave's stores; other waves write only positions it
  discards).
CPU only; nothing here runs on the GPU or calls the oracle."""
import random

import pytest

WAVE = 64


def _run_model(nb, head, q, order_seed=None):
    n_total = head + nb
    original = [1000.0 + k for k in range(n_total)]
    mem = list(original)
    writes = {}
    n4 = nb >> 2

    def rd(idx):
        assert 0 <= idx < n_total, ("read outside the array", nb, head, q, idx)
        return mem[idx]

    def wr(idx, val):
        assert 0 <= idx < n_total, ("write outside the array", nb, head, q, idx)
        assert idx not in writes, ("element written twice", nb, head, q, idx)
        writes[idx] = val
        mem[idx] = val

    chunks = list(range((n4 + WAVE - 1) // WAVE))
    if order_seed is not None:
        random.Random(order_seed).shuffle(chunks)
    for c in chunks:
        lanes = range(WAVE)
        i_ = [c * WAVE + lane for lane in lanes]
        ic_ = [min(i, n4 - 1) for i in i_]
        own_ = [lane == WAVE - 1 or ic_[lane] == n4 - 1 for lane in lanes]
        # loads: the aligned vector holding the lane's first element, or the
        # lane's elements of it one by one where it would start before the array
        a_ = []
        for lane in lanes:
            ic = ic_[lane]
            if ic == 0 and head < q:
                a = [None] * 4
                a[3] = rd(head + 3 - q)
                if q <= 2:
                    a[2] = rd(head + 2 - q)
                if q == 1:
                    a[1] = rd(head)
            else:
                base = head - q + 4 * ic
                a = [rd(base + k) for k in range(4)]
            a_.append(a)
        got = []
        for lane in lanes:
            a = a_[lane]
            nxt = a_[lane + 1] if lane + 1 < WAVE else a_[lane]  # shuffle down by one lane
            b = [nxt[0], nxt[1], nxt[2]]
            if own_[lane]:
                p = head + 4 * ic_[lane] + 4 - q
                b[0] = rd(p)
                if q >= 2:
                    b[1] = rd(p + 1)
                if q == 3:
                    b[2] = rd(p + 2)
            r = {1: [a[1], a[2], a[3], b[0]], 2: [a[2], a[3], b[0], b[1]],
                 3: [a[3], b[0], b[1], b[2]]}[q]
            if i_[lane] < n4:
                want = [original[head + 4 * i_[lane] + k] for k in range(4)]
                assert r == want, ("lane read the wrong elements", nb, head, q, lane)
            got.append([x + 0.5 if x is not None else None for x in r])  # the "update"
        # stores
        for lane in lanes:
            i = i_[lane]
            if i >= n4:
                continue
            r = got[lane]
            prev = got[lane - 1] if lane > 0 else got[lane]  # shuffle up by one lane
            p = head + 4 * i
            if lane != 0:
                x = {1: [prev[3], r[0], r[1], r[2]], 2: [prev[2], prev[3], r[0], r[1]],
                     3: [prev[1], prev[2], prev[3], r[0]]}[q]
                base = head - q + 4 * i
                for k in range(4):
                    wr(base + k, x[k])
            else:
                wr(p, r[0])
                if q <= 2:
                    wr(p + 1, r[1])
                if q == 1:
                    wr(p + 2, r[2])
            if own_[lane]:
                if q == 3:
                    wr(p + 1, r[1])
                    wr(p + 2, r[2])
                elif q == 2:
                    wr(p + 2, r[2])
                wr(p + 3, r[3])
    body = set(range(head, head + 4 * n4))
    assert set(writes) == body, ("body not covered exactly", nb, head, q)
    for k, val in writes.items():
        assert val == original[k] + 0.5, ("wrong value stored", nb, head, q, k)


BODIES = list(range(4, 140)) + [255, 256, 257, 4095, 4096, 4097, 4099, 8191, 12_800]


@pytest.mark.parametrize("q", [1, 2, 3])
@pytest.mark.parametrize("head", list(range(8)) + [60, 61, 62, 63])
def test_shifted_vectors_stay_in_bounds_and_cover_the_body(q, head):
    for nb in BODIES:
        _run_model(nb, head, q)


@pytest.mark.parametrize("q", [1, 2, 3])
def test_waves_in_any_order_see_only_values_from_before_the_stores(q):
    for seed, (nb, head) in enumerate([(4099, 0), (8191, 5), (12_800, 63), (257, 2), (70, 61)]):
        _run_model(nb, head, q, order_seed=seed)
