"""Pins for the oracle's g(s) search (CPU only).

The rule (ResearchPod summary, 2nd paragraph: distant positions are folded by the
least integer factor that keeps them inside the trained range) is checked against
the closed form ceil(s/L), against the range/minimality invariants it must
satisfy, and against hand-worked values for every workload size.
"""

import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "group_factor.txt")


def _golden_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                s, big_l, g = (int(x) for x in line.split())
                rows.append((s, big_l, g))
    return rows


@pytest.mark.parametrize("s,big_l,g", _golden_rows())
def test_golden_values(s, big_l, g):
    assert oracle.group_factor(s, big_l) == g


@pytest.mark.parametrize("big_l", [1, 2, 3, 7, 512])
def test_exhaustive_small(big_l):
    for s in range(1, 4 * big_l + 1):
        g = oracle.group_factor(s, big_l)
        assert g == max(1, -(-s // big_l))            # ceil(s / L)
        # range: every aliased position p // g, p < s, lies in 0..L-1
        assert (s - 1) // g <= big_l - 1
        # minimality: g - 1 would leave some position outside the window
        if g > 1:
            assert (s - 1) // (g - 1) > big_l - 1


def test_large_window_sampled():
    big_l = 32768
    rng = np.random.default_rng(7)
    for s in list(rng.integers(1, 4 * big_l + 1, size=200)) + [big_l - 1, big_l, big_l + 1, 2 * big_l,
                                                              2 * big_l + 1, 3 * big_l, 4 * big_l]:
        s = int(s)
        g = oracle.group_factor(s, big_l)
        assert g == max(1, -(-s // big_l))
        assert (s - 1) // g <= big_l - 1
        if g > 1:
            assert (s - 1) // (g - 1) > big_l - 1


def test_max_remote_distance_within_window():
    # The grouped branch only ever sees aliased distances a(p) - a(j) in 0..L-1.
    for s, big_l in [(2048, 512), (98304, 32768), (131072, 32768), (7, 3)]:
        g = oracle.group_factor(s, big_l)
        a = oracle.aliased_position(np.arange(s), g)
        assert a.max() - a.min() <= big_l - 1


def test_short_inputs_keep_base_model():
    # Abstract: the base model is recovered exactly at short inputs -> g == 1 for s <= L.
    for big_l in (1, 5, 512, 32768):
        for s in (1, big_l // 2 + 1, big_l):
            assert oracle.group_factor(s, big_l) == 1
        assert oracle.group_factor(big_l + 1, big_l) == 2


def test_invalid_arguments():
    with pytest.raises(ValueError):
        oracle.group_factor(0, 4)
    with pytest.raises(ValueError):
        oracle.group_factor(4, 0)
