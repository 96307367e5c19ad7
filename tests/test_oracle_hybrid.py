"""Pins of the hybrid-backbone transaction oracle (On-Demand Attention notes,
§2.3: recurrent and convolution states saved before the local trial,
restored before the full retry, only the chosen update committed; §3.3: the
recurrent layers keep their native computation).

* SiLU and the L2 normalisation against closed forms.
* The delta rule: a unit key written with alpha = beta = 1 reads back its
  value exactly; beta = 0 is pure decay; orthogonal keys keep separate
  values; the zero-state step has a closed form.
* The convolution: identity and pure-delay taps over several steps.
* The transaction: the committed state is the chosen candidate, the full
  candidate starts from the pre-step state (not from the local one), the
  caller's pre-step state is left untouched, and identical inputs give
  identical candidates.
"""
import math

import numpy as np
import pytest

from oracle import hybrid as HY
from oracle.oda_oracle import bf16_to_f64, f64_to_bf16


def test_delta_rule_reads_back_its_value():
    rng = np.random.default_rng(1)
    S = rng.normal(size=(6, 5))
    k = rng.normal(size=5)
    k /= np.linalg.norm(k)
    v = rng.normal(size=6)
    S2 = HY.delta_update(S, k, v, 1.0, 1.0)
    assert np.allclose(S2 @ k, v, atol=1e-12)
    # directions orthogonal to k are untouched
    u = rng.normal(size=5)
    u -= np.dot(u, k) * k
    assert np.allclose(S2 @ u, S @ u, atol=1e-12)


def test_delta_rule_decay_only_and_identity():
    rng = np.random.default_rng(2)
    S = rng.normal(size=(4, 4))
    k = rng.normal(size=4)
    v = rng.normal(size=4)
    assert np.allclose(HY.delta_update(S, k, v, 0.7, 0.0), 0.7 * S, atol=1e-14)
    assert np.array_equal(HY.delta_update(S, k, v, 1.0, 0.0), S)


def test_orthogonal_keys_keep_separate_values():
    S = np.zeros((3, 4))
    e1, e2 = np.eye(4)[0], np.eye(4)[2]
    v1, v2 = np.array([1.0, -2.0, 0.5]), np.array([0.25, 4.0, -1.0])
    S = HY.delta_update(S, e1, v1, 1.0, 1.0)
    S = HY.delta_update(S, e2, v2, 1.0, 1.0)
    assert np.allclose(S @ e1, v1) and np.allclose(S @ e2, v2)
    # overwriting e1 replaces its value (the delta rule, not accumulation)
    S = HY.delta_update(S, e1, v2, 1.0, 1.0)
    assert np.allclose(S @ e1, v2) and np.allclose(S @ e2, v2)


def _conv_weights(C, taps):
    w = np.zeros((C, 4))
    w[:, :] = taps
    return f64_to_bf16(w)


def test_convolution_identity_and_delay():
    C = 6
    xs = [f64_to_bf16(np.arange(C) + 10.0 * t) for t in range(6)]
    for taps, delay in (([0, 0, 0, 1], 0), ([1, 0, 0, 0], 3), ([0, 1, 0, 0], 2)):
        st = np.zeros((3, C))
        w = bf16_to_f64(_conv_weights(C, taps))
        for t, x in enumerate(xs):
            y, st = HY.conv_step(st, bf16_to_f64(x), w)
            want = bf16_to_f64(xs[t - delay]) if t >= delay else np.zeros(C)
            assert np.array_equal(y, want), (taps, t)
        assert np.array_equal(st, np.stack([bf16_to_f64(x) for x in xs[-3:]]))


def _layer_inputs(rng, H, d):
    C = 3 * H * d
    x = f64_to_bf16(rng.normal(size=C))
    w = f64_to_bf16(rng.normal(size=(C, 4)) * 0.5)
    alpha = rng.uniform(0.8, 1.0, size=H)
    beta = rng.uniform(0.1, 0.9, size=H)
    return x, w, alpha, beta


def test_silu_and_l2_norm_closed_forms():
    """SiLU(x) = x sigma(x): SiLU(0) = 0, SiLU(ln 3) = (3/4) ln 3 and
    SiLU(x) - SiLU(-x) = x.  The normalisation's epsilon sits inside the
    square root: a vector with |x|^2 = eps maps to x / sqrt(2 eps)."""
    assert HY.silu(np.float64(0.0)) == 0.0
    assert math.isclose(float(HY.silu(np.float64(math.log(3.0)))), 0.75 * math.log(3.0), rel_tol=1e-15)
    x = np.linspace(-6.0, 6.0, 25)
    assert np.allclose(HY.silu(x) - HY.silu(-x), x, rtol=0.0, atol=1e-14)
    e = HY.GDN_EPS
    v = np.array([math.sqrt(e), 0.0])
    assert np.allclose(HY.l2_normalise(v), v / math.sqrt(2.0 * e), rtol=1e-12, atol=0.0)
    assert np.array_equal(HY.l2_normalise(np.zeros(3)), np.zeros(3))


def test_zero_state_step_closed_form():
    rng = np.random.default_rng(3)
    H, d = 2, 8
    x, w, alpha, beta = _layer_inputs(rng, H, d)
    S0 = np.zeros((H, d, d))
    conv0 = np.zeros((3, 3 * H * d))
    o, S1, _ = HY.gdn_layer_step(S0, conv0, x, w, alpha, beta)
    a = HY.silu(bf16_to_f64(x) * bf16_to_f64(w)[:, 3])         # zero history: only the last tap
    for h in range(H):
        q = a[h * d:(h + 1) * d]
        k = a[H * d + h * d:H * d + (h + 1) * d]
        v = a[2 * H * d + h * d:2 * H * d + (h + 1) * d]
        qh, kh = q / math.sqrt(q @ q + 1e-6), k / math.sqrt(k @ k + 1e-6)
        assert np.allclose(S1[h], beta[h] * np.outer(v, kh), atol=1e-14)
        assert np.allclose(o[h], beta[h] * v * (kh @ qh) / math.sqrt(d), atol=1e-14)


def _random_state(rng, L, H, d):
    return HY.HybridState([rng.normal(size=(H, d, d)) * 0.3 for _ in range(L)],
                          [bf16_to_f64(f64_to_bf16(rng.normal(size=(3, 3 * H * d)))) for _ in range(L)])


def _branch_inputs(rng, L, H, d):
    return [(f64_to_bf16(rng.normal(size=3 * H * d)), rng.uniform(0.8, 1.0, size=H), rng.uniform(0.1, 0.9, size=H))
            for _ in range(L)]


def test_transaction_commits_the_chosen_candidate_from_the_pre_step_state():
    rng = np.random.default_rng(4)
    L, H, d = 3, 2, 8
    st = _random_state(rng, L, H, d)
    w = [f64_to_bf16(rng.normal(size=(3 * H * d, 4)) * 0.5) for _ in range(L)]
    loc, ful = _branch_inputs(rng, L, H, d), _branch_inputs(rng, L, H, d)
    before = st.copy()
    # local branch chosen
    out_l, out_f, new = HY.transaction_step(st, loc, ful, w, 0)
    assert out_f is None
    _, cand_l = HY.branch_pass(before, loc, w)
    for l in range(L):
        assert np.array_equal(new.S[l], cand_l.S[l]) and np.array_equal(new.conv[l], cand_l.conv[l])
    # the caller's state is the pre-step state still
    for l in range(L):
        assert np.array_equal(st.S[l], before.S[l]) and np.array_equal(st.conv[l], before.conv[l])
    # full branch chosen: its candidate starts from the pre-step state
    _, out_f, new_f = HY.transaction_step(st, loc, ful, w, 1)
    _, cand_f = HY.branch_pass(before, ful, w)
    out_dbl, dbl = HY.double_advance(before, loc, ful, w)
    for l in range(L):
        assert np.array_equal(new_f.S[l], cand_f.S[l])
        assert not np.allclose(new_f.S[l], dbl.S[l])           # advancing twice is detectably different
        assert not np.array_equal(new_f.conv[l], dbl.conv[l])
    assert not np.allclose(out_f[0], out_dbl[0])


def test_identical_inputs_give_identical_candidates():
    rng = np.random.default_rng(5)
    L, H, d = 2, 2, 8
    st = _random_state(rng, L, H, d)
    w = [f64_to_bf16(rng.normal(size=(3 * H * d, 4)) * 0.5) for _ in range(L)]
    loc = _branch_inputs(rng, L, H, d)
    out_l, out_f, new = HY.transaction_step(st, loc, loc, w, 1)
    for a, b in zip(out_l, out_f):
        assert np.array_equal(a, b)
