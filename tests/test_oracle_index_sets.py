"""Pins of the oracle's index sets (S^L, S^F) against the page's statements.

On-Demand Attention notes, section 2.1: S^F_t = {1..t};
S^L_t = {1..min(s,t)} U {max(1,t-w+1)..t} with s=4, w=2048, the window
including the current position, and the two sets first differing at
position 2053.
"""
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import full_index_set, local_index_set

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "index_sets.txt")


def _parse_missing(tok):
    if tok == "-":
        return set()
    out = set()
    for part in tok.split(","):
        if ".." in part:
            a, b = part.split("..")
            out |= set(range(int(a), int(b) + 1))
        else:
            out.add(int(part))
    return out


def _golden_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            s, w, t, size, miss = line.split()
            rows.append((int(s), int(w), int(t), int(size), _parse_missing(miss)))
    return rows


@pytest.mark.parametrize("s,w,t,size,missing", _golden_rows())
def test_golden_index_sets(s, w, t, size, missing):
    SL = local_index_set(t, s, w)
    SF = full_index_set(t)
    assert len(SL) == size
    one_based_missing = set((SF + 1).tolist()) - set((SL + 1).tolist())
    assert one_based_missing == missing
    assert np.all(np.diff(SL) > 0), "ascending, no duplicates"


def test_first_difference_is_2053():
    """The page: with s=4, w=2048 the trainable positions start at 2053."""
    first = None
    for t in range(1, 2100):
        if len(local_index_set(t)) != len(full_index_set(t)):
            first = t
            break
    assert first == 2053


def test_brute_membership_default_sizes():
    """Membership by the predicate 'in the sink or in the window' for every
    t up to 5000 (the page's s=4, w=2048)."""
    s, w = 4, 2048
    for t in list(range(1, 80)) + list(range(2040, 2070)) + list(range(4990, 5001)):
        brute = [i for i in range(1, t + 1) if i <= s or i >= t - w + 1]
        assert (local_index_set(t, s, w) + 1).tolist() == brute


def test_closed_form_size():
    for t in range(1, 6000, 7):
        assert len(local_index_set(t)) == min(t, 4 + 2048)
        assert len(full_index_set(t)) == t


def test_current_token_always_in_local_set():
    for t in (1, 2, 5, 2052, 2053, 9999):
        assert local_index_set(t)[-1] == t - 1


@settings(max_examples=200, deadline=None)
@given(s=st.integers(1, 9), w=st.integers(1, 40), t=st.integers(1, 120))
def test_property_small(s, w, t):
    SL = set((local_index_set(t, s, w) + 1).tolist())
    brute = {i for i in range(1, t + 1) if i <= s or i > t - w}
    assert SL == brute
    assert (SL == set(range(1, t + 1))) == (t <= s + w)
