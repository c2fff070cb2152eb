"""The split-KV plan's chunking rule (host restatement, no GPU): over random
row sets and edge cases, every row is tiled exactly once by its chunks,
every chunk index below the total is taken by exactly one workgroup of the
bound, the longer chunks go to the first half of the workgroups, forced
sizes give ceil(len / C) chunks, and the parity-dependent prefix equals a
scan of the maps "first parity -> chunks" composed in row order (the
associative form the kernel's wave scan uses).  The GPU tests check the
kernel's results against the oracle on layouts this rule chooses."""

import numpy as np
import pytest

from tests.helpers import (plan_chunk_of_workgroup, plan_chunk_range, plan_chunk_sizes, plan_first_chunks,
                           plan_row_counts)


def _compose(h, g):
    """h applied first, then g (maps parity p -> chunks)."""
    return tuple(h[p] + g[(p + h[p]) & 1] for p in (0, 1))


def _check_plan(lens, bound):
    big, small = plan_chunk_sizes(lens, bound)
    assert big >= small >= 384 and big - small in (0, 256)
    f = plan_first_chunks(lens, big, small)
    total = f[-1]
    assert total <= bound
    # the scan form: composing the per-row maps gives the same prefix
    acc = (0, 0)
    for x, fx in zip(lens, f[1:]):
        acc = _compose(acc, plan_row_counts(x, big, small))
        assert acc[0] == fx
    # every chunk index once, and every row entry exactly once
    cover = [np.zeros(int(x), np.int32) for x in lens]
    seen = set()
    for b in range(bound):
        j = plan_chunk_of_workgroup(b, bound, big, small)
        if j >= total:
            continue
        assert j not in seen
        seen.add(j)
        r = int(np.searchsorted(f, j, side="right")) - 1
        start, size = plan_chunk_range(f[r], j - f[r], big, small)
        end = min(start + size, int(lens[r]))
        assert 0 <= start < end <= lens[r]
        cover[r][start:end] += 1
        if big != small:
            assert (size == big) == (b < bound // 2)
    assert len(seen) == total
    for c in cover:
        assert np.all(c == 1)
    return big != small


def test_plan_rule_on_random_row_sets():
    rng = np.random.default_rng(7)
    skewed = checked = 0
    for _ in range(300):
        t = int(rng.integers(1, 300))
        bound = int(rng.choice([64, 128, 256, 512, 1024]))
        if t >= bound:
            continue
        lens = rng.integers(0, int(rng.choice([600, 5000, 200000])), t)
        if lens.sum() // t <= 512:
            continue
        skewed += _check_plan([int(x) for x in lens], bound)
        checked += 1
    assert checked > 100 and skewed > checked // 2


@pytest.mark.parametrize("lens, bound", [
    ([131072] * 8, 512),                  # rows that fill the bound exactly
    ([0, 5000, 0, 70000, 1], 512),        # empty and one-entry rows
    ([600] * 200, 512),                   # rows of barely more than one chunk
    ([100000] * 200, 512),
    ([513] * 255, 512),
    ([9000] + [0] * 63, 512),             # one row with every chunk
])
def test_plan_rule_edge_cases(lens, bound):
    _check_plan(lens, bound)


def test_forced_and_single_sizes_count_ceil():
    for length in (0, 1, 63, 64, 65, 640, 641, 100000):
        for c in (64, 128, 640, 2048):
            k0, k1 = plan_row_counts(length, c, c)
            assert k0 == k1 == -(-length // c)
