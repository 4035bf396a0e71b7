"""CPU model of the packed persistent schedule (fa_device.h: packed_units,
packed_schedule_build, packed_schedule_item): over all work-groups, every
(sequence, head, query tile) comes out exactly once, for causal / non-causal
calls, with and without a window; and under a causal window the units of a
sequence carry equal work, so the ranked list decreases."""
import random

import pytest

ROWS = 256
INT_MAX = 0x7FFFFFFF


def units_of(nt, fcap):
    f = min(fcap, nt)
    return nt - f + (f + 1) // 2


def build(lengths, heads, causal, window):
    key = [max(0, n + ROWS - 1) // ROWS for n in lengths]
    order = sorted(range(len(key)), key=lambda i: (-key[i], i))
    fcap = 0
    if causal:
        fcap = min(INT_MAX, (window - 1 + ROWS - 1) // ROWS) if window > 0 else INT_MAX
    first, acc = [], 0
    for r in range(len(key)):
        first.append(acc)
        acc += heads * units_of(key[order[r]], fcap)
    first.append(acc)
    return dict(key=key, order=order, first=first, units=acc, fcap=fcap, heads=heads, nseq=len(key))


def item(ps, i, causal, block, grid):
    slot = (block % 8) * (grid // 8) + block // 8
    lap, e = i >> 2, i & 3
    k0 = lap * 2 * grid
    if k0 >= ps["units"]:
        return -1, None
    k = k0 + (slot if (e >> 1) == 0 else 2 * grid - 1 - slot)
    if k >= ps["units"]:
        return 0, None
    lo, hi = 0, ps["nseq"]
    while hi - lo > 1:
        mid = (lo + hi) >> 1
        if ps["first"][mid] <= k:
            lo = mid
        else:
            hi = mid
    seq = ps["order"][lo]
    nt = ps["key"][seq]
    f = min(ps["fcap"], nt)
    per = nt - f + (f + 1) // 2
    local = k - ps["first"][lo]
    u, h = local % per, local // per
    if u < nt - f:
        if e & 1:
            return 0, None
        return 1, (seq, h, nt - 1 - u if causal else u)
    j = u - (nt - f)
    hi_t = f - 1 - j
    if e & 1:
        if hi_t == j:
            return 0, None
        return 1, (seq, h, j)
    return 1, (seq, h, hi_t)


def run(lengths, heads, causal, window, grid):
    ps = build(lengths, heads, causal, window)
    got = []
    for block in range(grid):
        i = 0
        while True:
            st, it = item(ps, i, causal, block, grid)
            if st < 0:
                break
            if st:
                got.append(it)
            i += 1
    want = [(s, h, t) for s, n in enumerate(lengths) for h in range(heads) for t in range((n + ROWS - 1) // ROWS)]
    return ps, got, want


CASES = [
    ([6096, 518, 1431, 1511, 1999, 1575, 6342, 3435, 3192, 5279, 1390], 28),  # the 32k packed workload
    ([1, 255, 256, 257, 8192], 3),
    ([4096] * 8, 2),
    ([0, 300, 0, 5000], 4),
    ([100], 1),
]


@pytest.mark.parametrize("lengths,heads", CASES)
@pytest.mark.parametrize("causal,window", [(True, 0), (True, 4096), (True, 1), (True, 300), (True, 10 ** 9),
                                           (False, 0), (False, 4096)])
@pytest.mark.parametrize("grid", [8, 256])
def test_every_tile_once(lengths, heads, causal, window, grid):
    ps, got, want = run(lengths, heads, causal, window, grid)
    assert sorted(got) == sorted(want)
    assert len(got) == len(set(got))


def test_random_lengths():
    rng = random.Random(7)
    for _ in range(40):
        lengths = [rng.randint(1, 9000) for _ in range(rng.randint(1, 20))]
        heads = rng.randint(1, 6)
        window = rng.choice([0, 1, 64, 700, 4096, 20000])
        causal = rng.random() < 0.8
        grid = rng.choice([8, 64, 256])
        _, got, want = run(lengths, heads, causal, window, grid)
        assert sorted(got) == sorted(want)


def key_tiles(n, qt, window):
    """64-key tiles a causal query tile qt of a sequence of n visits (window 0: none)."""
    q0, q1 = qt * ROWS, min(qt * ROWS + ROWS, n) - 1
    lo = max(0, q0 - window + 1) if window > 0 else 0
    return (q1 + 1 + 63) // 64 - lo // 64


@pytest.mark.parametrize("window", [0, 4096, 1000])
def test_units_of_a_sequence_carry_equal_work(window):
    """Full tiles and pairs of partial tiles see the same number of key tiles (up to
    the sequence's last, shorter tile and the middle tile of an odd count)."""
    ps = build([8192, 5000], 1, True, window)
    for s_, n in enumerate([8192, 5000]):
        nt = ps["key"][s_]
        f = min(ps["fcap"], nt)
        work = [key_tiles(n, qt, window) for qt in range(f, nt - 1)]
        work += [key_tiles(n, f - 1 - j, window) + key_tiles(n, j, window) for j in range(f // 2)]
        assert max(work) - min(work) <= 5, (window, n, work)

