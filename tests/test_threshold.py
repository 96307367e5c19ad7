"""Host logic that turns a target call rate into the rule's threshold
(step.tune_theta, step.match_rate), checked on the CPU against model
trajectories whose scores fall once a sequence has taken the full branch,
as the head's do when its hidden state changes branch."""
import math

import numpy as np
import pytest

from conditional_sparse_attention_amd.step import match_rate, tune_theta


def test_tune_theta_counts_and_edges():
    sc = np.array([3.0, -1.0, 2.0, 0.5, 1.0, -2.0, 0.0, 4.0])
    for rate, k in ((0.125, 1), (0.25, 2), (0.5, 4), (0.75, 6)):
        theta = tune_theta(sc, rate)
        assert int(np.count_nonzero(sc > theta)) == k   # the strict rule q > theta
    assert tune_theta(sc, 0.0) == math.inf and tune_theta(sc, 1.0) == -math.inf


def drifting(seed, steps=128, batch=4, pull=0.3):
    base = np.random.default_rng(seed).normal(size=(steps, batch))

    def run_pass(theta):
        sc = np.zeros_like(base)
        fl = np.zeros(base.shape, np.uint8)
        drift = np.zeros(batch)
        for j in range(steps):
            sc[j] = base[j] - pull * drift
            fl[j] = sc[j] > theta
            drift = 0.9 * drift + fl[j]
        return sc, fl

    return run_pass


@pytest.mark.parametrize("rate", [0.0, 0.125, 0.25, 0.416, 1.0])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_match_rate_reaches_the_target_on_its_own_trajectory(rate, seed):
    run_pass = drifting(seed)
    theta0 = tune_theta(run_pass(math.inf)[0], rate)
    n0 = int(np.count_nonzero(run_pass(theta0)[1]))
    theta, n, k, passes = match_rate(run_pass, theta0, rate, max_passes=12)
    assert k == round(rate * 512)
    assert int(np.count_nonzero(run_pass(theta)[1])) == n    # the returned theta reproduces its count
    assert abs(n - k) <= abs(n0 - k)                          # never worse than the all-local threshold
    # the count moves with the trajectory, so it may stop one decision short
    assert abs(n - k) <= 1, (rate, seed, n, k, passes)
    assert 1 <= passes <= 12


def test_match_rate_stops_at_max_passes_with_the_closest_pass():
    calls = []
    run = drifting(5)

    def run_pass(theta):
        calls.append(theta)
        return run(theta)

    theta0 = tune_theta(run(math.inf)[0], 0.47)
    theta, n, k, passes = match_rate(run_pass, theta0, 0.47, max_passes=2)
    assert passes == 2 and len(calls) == 2 and theta in calls
    counts = [int(np.count_nonzero(run(t)[1])) for t in calls]
    assert abs(n - k) == min(abs(c - k) for c in counts)
