"""Pins for the oracle's integer side: window restriction and Split-KV ranges (CPU only)."""

import json
import os
import random

import numpy as np
import pytest

from oracle import restrict_to_window, split_page_ranges, visible_range, window_start_page, window_table_width

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cases():
    return json.load(open(os.path.join(GOLDEN, "window_cases.json")))


@pytest.mark.parametrize("case", _cases()["cases"], ids=lambda c: f"L{c['L']}_w{c['w']}_sq{c['sq']}")
def test_window_hand_worked(case):
    L, w, sq, P = case["L"], case["w"], case["sq"], case["P"]
    assert window_start_page(L, w, sq, P) == case["start_page"]
    assert window_table_width(w, sq, P, 10**6) == case["width"]
    lens, _ = restrict_to_window([L], np.zeros((1, -(-L // P) or 1), np.int32), w, sq, P)
    assert int(lens[0]) == case["L_restricted"]


@pytest.mark.parametrize("case", _cases()["table_cases"])
def test_window_table_gather_hand_worked(case):
    tab = np.array([case["table"]], np.int32)
    _, out = restrict_to_window([case["L"]], tab, case["w"], case["sq"], case["P"])
    assert out[0].tolist() == case["restricted"]


def test_window_is_smallest_page_aligned_cover():
    """Property from the page's prose: the visible start is page aligned, covers the
    window suffix [L - w - sq + 1, L), and adds at most P - 1 tokens in front."""
    rng = random.Random(3)
    for _ in range(20000):
        P = rng.choice([1, 8, 16, 64])
        w = rng.randint(1, 300)
        sq = rng.randint(1, 20)
        L = rng.randint(0, 1000)
        start, end = visible_range(L, w, sq, P)
        assert end == L
        assert start % P == 0 and start >= 0
        need = L - w - sq + 1
        if need <= 0:
            assert start == 0
        else:
            assert start <= need < start + P


def test_no_window_is_identity():
    lens = np.array([5, 17, 300])
    tab = np.arange(3 * 20, dtype=np.int32).reshape(3, 20)
    l2, t2 = restrict_to_window(lens, tab, 0, 4, 16)
    assert l2.tolist() == lens.tolist() and np.array_equal(t2, tab)
    assert visible_range(300, 0, 4, 16) == (0, 300)


def test_restricted_table_reaches_the_same_keys():
    """Keys addressed through (restricted table, restricted length) are the original
    keys [start, L) in order."""
    rng = random.Random(4)
    for _ in range(300):
        P = rng.choice([4, 16])
        sq = rng.randint(1, 8)
        w = rng.randint(1, 80)
        L = rng.randint(1, 200)
        W = -(-L // P) + rng.randint(0, 3)
        tab = np.array([rng.sample(range(1000), W)], np.int32)
        l2, t2 = restrict_to_window([L], tab, w, sq, P)
        start, _ = visible_range(L, w, sq, P)
        orig = [(int(tab[0, j // P]), j % P) for j in range(start, L)]
        restr = [(int(t2[0, j // P]), j % P) for j in range(int(l2[0]))]
        assert orig == restr


@pytest.mark.parametrize("n", [0, 1, 5, 16, 17, 513])
@pytest.mark.parametrize("S", [1, 2, 3, 16, 64])
def test_split_ranges_partition(n, S):
    r = split_page_ranges(n, S)
    assert len(r) == S
    cur = 0
    per = -(-n // S) if n else 0
    for first, count in r:
        assert count >= 0 and count <= per
        if count:
            assert first == cur
        cur += count
    assert cur == n


def _compositions(n, S):
    """Every way to cut n pages into S in-order chunks (sizes >= 0)."""
    if S == 1:
        yield (n,)
        return
    for first in range(n + 1):
        for rest in _compositions(n - first, S - 1):
            yield (first,) + rest


@pytest.mark.parametrize("S", [1, 2, 3, 4, 5])
def test_split_ranges_brute_force(S):
    # Reading R9 as a selection over all cuts: the smallest possible largest chunk
    # (equal chunks), filled front to back (trailing chunks absorb the shortfall).
    for n in range(0, 13):
        cuts = list(_compositions(n, S))
        best = min(max(c) for c in cuts)
        chosen = max(c for c in cuts if max(c) == best)  # lexicographically largest
        got = split_page_ranges(n, S)
        assert tuple(count for _, count in got) == chosen, (n, S)
        firsts = [0]
        for c in chosen[:-1]:
            firsts.append(firsts[-1] + c)
        assert [first for first, count in got if count] == [f for f, c in zip(firsts, chosen) if c]

