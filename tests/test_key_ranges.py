"""Host model of the GQA decode's key-range cut (no GPU).

The split kernel and the merge kernel find a request's pieces independently
from seq_lens; this restates both lookups in Python and checks, on random
batches, that they agree: every tile of every request is walked exactly
once, partial slots g + b are distinct and below K + batch, the merge reads
exactly the pieces the split kernel wrote, and a request is written final
exactly when it lies inside one range. It checks the arithmetic, not the
device code; the GPU tests compare the device code with the oracle.
"""

import random

import pytest


def request_tiles(lk, q_len, window_left):
    base = (max(0, lk - q_len - window_left) & ~31) if window_left >= 0 else 0
    return max(1, (lk - base + 31) >> 5)


def split_kernel_pieces(lens, q_len, wl, key_ranges):
    """(g, b, s0, s1, final, slot) of every piece, as the waves of each range walk them."""
    n = [request_tiles(x, q_len, wl) for x in lens]
    total = sum(n)
    ranges = min(key_ranges, total)
    out = []
    for g in range(key_ranges):
        if g >= ranges:
            continue
        t_lo, t_hi = g * total // ranges, (g + 1) * total // ranges
        # the request holding tile t_lo: first b whose inclusive prefix exceeds t_lo
        incl, b, p = 0, 0, 0
        for i, x in enumerate(n):
            incl += x
            if incl > t_lo:
                b, p = i, incl - x
                break
        while p < t_hi:
            s0, s1 = max(t_lo, p) - p, min(t_hi, p + n[b]) - p
            out.append((g, b, s0, s1, s0 == 0 and s1 == n[b], g + b))
            p += n[b]
            b += 1
    return out, n, total, ranges


def merge_pieces(lens, q_len, wl, key_ranges, b):
    n = [request_tiles(x, q_len, wl) for x in lens]
    total = sum(n)
    ranges = min(key_ranges, total)
    below = sum(n[:b])
    g_first = ((below + 1) * ranges - 1) // total
    g_last = ((below + n[b]) * ranges - 1) // total
    return [g + b for g in range(g_first, g_last + 1)]


@pytest.mark.parametrize("seed", range(40))
def test_cut_covers_every_tile_once_and_merge_finds_the_pieces(seed):
    rng = random.Random(seed)
    batch = rng.choice([1, 2, 3, 17, 64, 200, 512])
    hi = rng.choice([1, 40, 300, 8192])
    lens = [rng.choice([0, rng.randint(0, hi)]) if rng.random() < 0.2 else rng.randint(0, hi) for _ in range(batch)]
    q_len = rng.randint(1, 4)
    wl = rng.choice([-1, -1, 0, 50, 1000])
    k = rng.choice([1, 2, 7, 384, 512])
    pieces, n, total, ranges = split_kernel_pieces(lens, q_len, wl, k)
    # every tile of every request exactly once
    cover = [[0] * x for x in n]
    for g, b, s0, s1, fin, slot in pieces:
        assert 0 <= s0 < s1 <= n[b]
        for t in range(s0, s1):
            cover[b][t] += 1
    assert all(c == 1 for row in cover for c in row)
    # slots distinct and inside the workspace's K + batch rows per request row
    slots = [p[5] for p in pieces if not p[4]]
    assert len(slots) == len(set(slots)) and all(0 <= s < k + batch for s in slots)
    # ranges are as even as integers allow
    sizes = [(g + 1) * total // ranges - g * total // ranges for g in range(ranges)]
    assert max(sizes) - min(sizes) <= 1 and min(sizes) >= 1
    for b in range(batch):
        mine = [p for p in pieces if p[1] == b]
        found = merge_pieces(lens, q_len, wl, k, b)
        if len(mine) == 1:
            assert mine[0][4] and len(found) == 1          # final, left alone by the merge
        else:
            assert not any(p[4] for p in mine)
            assert found == [p[5] for p in mine]           # in walk order


def test_request_tiles_follow_the_window():
    assert request_tiles(0, 1, -1) == 1          # an empty request still owns one (empty) tile
    assert request_tiles(32, 1, -1) == 1 and request_tiles(33, 1, -1) == 2
    # window: keys from the tile holding lk - q_len - window_left
    assert request_tiles(1000, 4, 100) == -(-(1000 - ((1000 - 4 - 100) & ~31)) // 32)
    assert request_tiles(50, 4, 1000) == 2       # a window wider than the history
