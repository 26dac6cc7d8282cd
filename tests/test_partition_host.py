"""The balanced split-K partition of the GQA decode, checked on the host (no GPU).

The decode kernel lists every 128-token tile of every (sequence, KV head) unit in the order
u = b * Hkv + kvh and gives wave i of W the tiles [floor(i T / W), floor((i + 1) T / W));
a wave writes one partial per unit its range touches, into slot i + u, and the merge finds
a unit's partials from the waves that own its first and last tiles, with the closed form
owner(x) = ceil((x + 1) W / T) - 1.  These tests check, on many batches, the properties the
kernels rely on: the ranges cover every tile exactly once, owner() inverts them, the slots
of one unit are consecutive and no two (wave, unit) pairs share a slot (so W + U slots
suffice).  The wave count W is the library's own plan, read through its host functions.
"""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from fp4_kv_cache_amd import lib as L  # noqa: E402


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from fp4_kv_cache_amd import build
        build.build()
    return L.load()


def owner(x, total, waves):
    return ((x + 1) * waves + total - 1) // total - 1


def shares(total, waves):
    return [(i * total // waves, (i + 1) * total // waves) for i in range(waves)]


def planned_waves(lens, hkv, page):
    c = L.FP4KVCache(0, 0, 1 << 20, page, hkv, 128, 0, max(len(lens), 1))
    maxlen = max(int(np.max(lens)) if len(lens) else 0, 1)
    words = L.fp4kv_cache_read_sink_words(c, len(lens), 4 * hkv, maxlen)
    assert words > 0 and words % 64 == 0
    return words // 64


def device_waves(total, planned):
    # the kernels shrink the plan to no more shares than tiles
    return min(planned, total)


def check_partition(lens, hkv, page):
    tiles = [-(-int(n) // 128) for n in lens]
    units = [(b, h) for b in range(len(lens)) for h in range(hkv)]
    unit_tiles = [tiles[b] for b, _ in units]
    total = sum(unit_tiles)
    waves = device_waves(total, planned_waves(lens, hkv, page))
    if total == 0:
        assert waves == 0
        return
    rng = shares(total, waves)
    # every tile in exactly one share, shares contiguous and in order
    assert rng[0][0] == 0 and rng[-1][1] == total
    for (a0, a1), (b0, b1) in zip(rng, rng[1:]):
        assert a1 == b0 and a0 < a1
    # owner() inverts the shares
    for i, (x0, x1) in enumerate(rng):
        for x in (x0, x1 - 1, (x0 + x1) // 2):
            assert owner(x, total, waves) == i
    # slots: wave i writes unit u's partial into slot i + u
    start = np.concatenate([[0], np.cumsum(unit_tiles)])
    used = {}
    for u, n in enumerate(unit_tiles):
        if n == 0:
            continue
        first, last = owner(start[u], total, waves), owner(start[u + 1] - 1, total, waves)
        slots = [i + u for i in range(first, last + 1)]
        # the waves first..last are exactly those whose ranges meet the unit's tiles
        assert rng[first][0] <= start[u] < rng[first][1]
        assert rng[last][0] <= start[u + 1] - 1 < rng[last][1]
        for s in slots:
            assert s not in used, "slot %d used by units %d and %d" % (s, used[s], u)
            used[s] = u
            assert 0 <= s < waves + len(units)


@pytest.mark.parametrize("lens,hkv,page", [
    ([32768] * 16, 8, 64),                                     # the Qwen3-4B batch
    ([131072] * 4, 8, 64),                                     # long context
    ([1, 0, 130, 600, 0, 0, 257, 64, 1000, 5, 0, 385], 8, 64),  # shares crossing units
    ([0, 0, 0], 8, 64),                                        # nothing to do
    ([4096], 2, 16),                                           # the tiny configuration
])
def test_partition_fixed_batches(lib, lens, hkv, page):
    check_partition(np.array(lens), hkv, page)


def test_partition_random_ragged_batches(lib):
    rng = np.random.default_rng(11)
    for _ in range(60):
        batch = int(rng.integers(1, 90))
        hkv = int(rng.choice([1, 2, 4, 8]))
        lens = rng.integers(0, 70000, size=batch)
        lens[rng.random(batch) < 0.2] = 0
        check_partition(lens, hkv, int(rng.choice([32, 64, 128])))
