"""CPU model of the packed persistent schedule (fa_device.h: packed_schedule_build,
packed_schedule_item): over all work-groups, every (sequence, head, query tile)
comes out exactly once, for causal / non-causal calls, with and without a window,
and the unit order under a causal window decreases in work level by level."""
import random

import pytest

ROWS = 256
LEVELS_MAX = 512


def build(lengths, heads, causal, window):
    pair = causal and window <= 0
    key = [max(0, n + ROWS - 1) // ROWS for n in lengths]
    order = sorted(range(len(key)), key=lambda i: (-key[i], i))
    f = 0
    w = window if causal else 0
    if w > 0 and not pair:
        f = (w - 1 + ROWS - 1) // ROWS
    maxnt = key[order[0]] if key else 0
    nlev = min(f, maxnt)
    if nlev > LEVELS_MAX:
        f = nlev = 0
    first, acc = [], 0
    for r in range(len(key)):
        first.append(acc)
        nt = key[order[r]]
        acc += heads * ((nt + 1) // 2 if pair else max(0, nt - f))
    first.append(acc)
    full = acc
    lfirst, c = [], 0
    for lv in range(nlev):
        qt = nlev - 1 - lv
        while c < len(key) and key[order[c]] > qt:
            c += 1
        lfirst.append(acc)
        acc += heads * c
    lfirst.append(acc)
    return dict(key=key, order=order, first=first, lfirst=lfirst, full=full, units=acc, f=f, nlev=nlev,
                heads=heads, pair=pair, nseq=len(key))


def item(ps, i, causal, block, grid):
    slot = (block % 8) * (grid // 8) + block // 8
    lap, e = i >> 2, i & 3
    k0 = lap * 2 * grid
    if k0 >= ps["units"]:
        return -1, None
    k = k0 + (slot if (e >> 1) == 0 else 2 * grid - 1 - slot)
    if k >= ps["units"]:
        return 0, None
    if k >= ps["full"]:
        if e & 1:
            return 0, None
        lo, hi = 0, ps["nlev"]
        while hi - lo > 1:
            mid = (lo + hi) >> 1
            if ps["lfirst"][mid] <= k:
                lo = mid
            else:
                hi = mid
        j = k - ps["lfirst"][lo]
        return 1, (ps["order"][j // ps["heads"]], j % ps["heads"], ps["nlev"] - 1 - lo)
    lo, hi = 0, ps["nseq"]
    while hi - lo > 1:
        mid = (lo + hi) >> 1
        if ps["first"][mid] <= k:
            lo = mid
        else:
            hi = mid
    seq = ps["order"][lo]
    nt = ps["key"][seq]
    per = (nt + 1) // 2 if ps["pair"] else nt - ps["f"]
    local = k - ps["first"][lo]
    u, h = local % per, local // per
    heavy = nt - 1 - u if causal else ps["f"] + u
    if e & 1:
        if not ps["pair"] or heavy == nt - 1 - heavy:
            return 0, None
        return 1, (seq, h, nt - 1 - heavy)
    return 1, (seq, h, heavy)


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


def _work(n, qt, window):
    q0, q1 = qt * ROWS, min(qt * ROWS + ROWS, n) - 1
    lo = max(0, q0 - window + 1)
    return (q1 + 1 + 63) // 64 - lo // 64


def test_level_order_decreases_in_work():
    lengths, heads, window = CASES[0][0], 28, 4096
    ps = build(lengths, heads, True, window)
    assert ps["f"] == 16 and ps["nlev"] == 16
    # the partial levels, in order, carry non-increasing work
    level_work = []
    for lv in range(ps["nlev"]):
        qt = ps["nlev"] - 1 - lv
        seqs = [ps["order"][r] for r in range((ps["lfirst"][lv + 1] - ps["lfirst"][lv]) // heads)]
        level_work.append(max(_work(lengths[s_], qt, window) for s_ in seqs))
    assert all(level_work[i] >= level_work[i + 1] for i in range(len(level_work) - 1))
    # every full tile but a sequence's last (shorter) one carries at least as
    # much work as the heaviest partial tile
    for s_, n in enumerate(lengths):
        for qt in range(ps["f"], (n + ROWS - 1) // ROWS - 1):
            assert _work(n, qt, window) >= level_work[0]
