"""Pins of the branch rule, the labels / Huber loss, the full-branch work
list and the commit (On-Demand Attention notes, sections 2.2 and 2.3)."""
import math
import os

import numpy as np
import pytest

from oracle import (benefit_label, branch_rule, commit, full_worklist, huber,
                    huber_loss, label_valid)

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLD, name)) as f:
        return [l.split() for l in f if l.strip() and not l.startswith("#")]


@pytest.mark.parametrize("row", _rows("rule.txt"))
def test_rule_hand_table(row):
    q, theta, force, want = float(row[0]), float(row[1]), int(row[2]), int(row[3])
    assert branch_rule(q, theta, force) == want


def test_rule_negative_zero_bits():
    assert branch_rule(float(np.float32(-0.0)), 0.0) == 0


@pytest.mark.parametrize("row", [r for r in _rows("labels.txt") if r[0] == "label"])
def test_label_hand_values(row):
    _, g, lam, want = row
    assert abs(benefit_label(float(g), float(lam)) - float(want)) < 1e-12


@pytest.mark.parametrize("row", [r for r in _rows("labels.txt") if r[0] == "huber"])
def test_huber_hand_values(row):
    _, r, want = row
    assert huber(float(r)) == float(want)


def test_huber_continuous_at_one():
    assert abs(huber(1.0 - 1e-12) - huber(1.0 + 1e-12)) < 1e-11


def test_label_is_monotone_and_odd():
    xs = np.linspace(-5, 5, 201)
    ys = [benefit_label(x) for x in xs]
    assert all(b > a for a, b in zip(ys, ys[1:]))
    for x in xs:
        assert benefit_label(-x) == -benefit_label(x)


def test_huber_loss_mean_over_valid_set():
    q = [0.0, 1.0, 3.0, 10.0]
    y = [0.5, 0.0, 0.0, float("nan")]
    valid = [label_valid(t, g) for t, g in zip([2053, 3000, 5000, 6000], y)]
    assert valid == [True, True, True, False]
    assert huber_loss(q, y, valid) == pytest.approx((0.125 + 0.5 + 2.5) / 3)
    assert not label_valid(2052, 0.1)


def test_worklist_brute_force():
    rng = np.random.default_rng(0)
    for _ in range(50):
        B = int(rng.integers(1, 33))
        flags = rng.integers(0, 2, size=B)
        pos = rng.integers(0, 5000, size=B)
        chunk = int(rng.choice([64, 256, 1000]))
        nsplit = [math.ceil((p + 1) / chunk) for p in pos]
        items = full_worklist(flags, nsplit)
        brute = [(b, s) for b in range(B) for s in range(10000)
                 if flags[b] and s * chunk < pos[b] + 1]
        assert items == brute
        assert len(items) == sum(int(f) * n for f, n in zip(flags, nsplit))
        # with lengths: the same pairs, each sequence's splits contiguous and
        # in order, sequences longest unit first (ties: ascending b)
        t = pos + 1
        nsplit = [int(rng.integers(1, 33)) for _ in range(B)]
        items = full_worklist(flags, nsplit, t)
        assert sorted(items) == [(b, s) for b in range(B) if flags[b] for s in range(nsplit[b])]
        order = [b for i, (b, s) in enumerate(items) if s == 0]
        for i, (b, s) in enumerate(items):
            assert s == 0 or items[i - 1] == (b, s - 1)
        unit = lambda b: -(-int(t[b]) // nsplit[b])
        for x, y in zip(order, order[1:]):
            assert unit(x) > unit(y) or (unit(x) == unit(y) and x < y)


def test_commit_invariants():
    rng = np.random.default_rng(1)
    L, B, H, T, d, D = 3, 4, 2, 10, 8, 16
    K = rng.integers(0, 65535, size=(L, B, H, T, d)).astype(np.uint16)
    V = rng.integers(0, 65535, size=(L, B, H, T, d)).astype(np.uint16)
    pos = np.array([0, 3, 7, 9])
    flags = [1, 0, 1, 0]
    kL, vL, kF, vF = (rng.integers(0, 65535, size=(L, B, H, d)).astype(np.uint16) for _ in range(4))
    oL, oF = (rng.integers(0, 65535, size=(B, D)).astype(np.uint16) for _ in range(2))
    K2, V2, pos2, h = commit(K, V, pos, flags, kL, vL, kF, vF, oL, oF)
    assert np.array_equal(pos2, pos + 1)
    for b in range(B):
        p = pos[b]
        ck, cv, co = (kF, vF, oF) if flags[b] else (kL, vL, oL)
        assert np.array_equal(K2[:, b, :, p], ck[:, b])
        assert np.array_equal(V2[:, b, :, p], cv[:, b])
        assert np.array_equal(h[b], co[b])
        mask = np.ones(T, bool)
        mask[p] = False
        assert np.array_equal(K2[:, b, :, mask], K[:, b, :, mask])
        assert np.array_equal(V2[:, b, :, mask], V[:, b, :, mask])
