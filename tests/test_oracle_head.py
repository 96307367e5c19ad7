"""Pins of the oracle's recall head R_psi (On-Demand Attention notes,
section 2.2: q_t = R_psi(h_{t-1}, E(x_t), h_t^L); three independent towers of
norm, projection and activation to 1024 dims; a 9216-dim interaction of the
raw vectors, pairwise products and pairwise absolute differences; projection
with residual fusion; two residual gated FFN blocks; scalar output; fp32;
28,325,889 parameters).

Each component is pinned by hand values; the composition by the page's
parameter count, by special weights with closed-form outputs, by routing of
each input to its own tower, and by symmetry / scale invariances.
"""
import math
import os

import numpy as np
import pytest

import synth
from oracle import (gated_ffn_block, head_layout, head_param_count, interaction,
                    recall_score, rms_norm, silu, unpack_head)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "head_shape.txt")


def _golden_shape():
    with open(GOLDEN) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                return [int(x) for x in line.split()]


def test_param_count_matches_page():
    hidden, tower, inter, count = _golden_shape()
    assert head_param_count(hidden, tower) == count
    lay = dict(head_layout(hidden, tower))
    assert lay["W_I"][1] == inter
    assert lay["W_H"] == (tower, hidden)


def test_layout_agrees_with_generator_format():
    """The packed blob format is defined three times (generator, oracle,
    HIP library); the generator's and the oracle's must agree."""
    for D in (2048, 4096):
        ours = [(n, s) for n, s in head_layout(D)]
        gens = [(n, s) for n, s, _ in synth.head_tensor_shapes(D)]
        assert ours == gens


def test_interaction_hand_values():
    a = np.array([1.0, 2.0])
    b = np.array([3.0, -1.0])
    c = np.array([0.0, 5.0])
    want = [1, 2, 3, -1, 0, 5, 3, -2, 0, 10, 0, -5, 2, 3, 1, 3, 3, 6]
    assert interaction(a, b, c).tolist() == want


def test_rms_norm_hand_values():
    x = np.array([3.0, 4.0])
    # mean of squares 12.5, sqrt = 3.5355339059327378
    np.testing.assert_allclose(rms_norm(x, np.ones(2), eps=0.0),
                               [0.8485281374238570, 1.1313708498984760], rtol=1e-15)
    np.testing.assert_allclose(rms_norm(x, np.array([2.0, -0.5]), eps=0.0),
                               [1.6970562748477140, -0.5656854249492380], rtol=1e-15)
    assert np.array_equal(rms_norm(np.zeros(4), np.ones(4)), np.zeros(4))


def test_silu_textbook_values():
    np.testing.assert_allclose(silu(np.array([0.0, 1.0, -1.0, 20.0, -40.0])),
                               [0.0, 0.7310585786300049, -0.2689414213699951,
                                19.999999958776927, -1.6993417021166355e-16], rtol=1e-14, atol=1e-300)


def test_gated_ffn_roles():
    """Zero gate -> identity; identity gate with a one-entry up projection
    and a non-symmetric down projection gives a closed form that changes if
    gate/up are swapped or down is transposed."""
    u = np.array([3.0, 4.0])
    g1 = np.ones(2)
    Z = np.zeros((2, 2))
    assert np.array_equal(gated_ffn_block(u, g1, Z, np.eye(2), np.eye(2)), u)
    Wg = np.eye(2)
    Wu = np.array([[0.0, 0.0], [1.0, 0.0]])
    Wd = np.array([[0.0, 1.0], [0.0, 2.0]])
    r = u / math.sqrt(12.5 + 1e-6)
    prod2 = r[1] / (1.0 + math.exp(-r[1])) * r[0]
    want = np.array([3.0 + prod2, 4.0 + 2.0 * prod2])
    np.testing.assert_allclose(gated_ffn_block(u, g1, Wg, Wu, Wd), want, rtol=1e-14)
    swapped = gated_ffn_block(u, g1, Wu, Wg, Wd)
    transposed = gated_ffn_block(u, g1, Wg, Wu, Wd.T)
    assert not np.allclose(swapped, want) and not np.allclose(transposed, want)


def _zero_params(D=2, T=2, F=2):
    return {n: np.zeros(s) for n, s in head_layout(D, T, F)}


def test_zero_weights_give_output_bias():
    P = _zero_params(8, 4, 6)
    P["c_o"] = np.array([0.375])
    rng = np.random.default_rng(0)
    q = recall_score(P, rng.normal(size=8), rng.normal(size=8), rng.normal(size=8))
    assert q == 0.375


def test_residual_fusion_closed_form():
    """Projection weights zero, tower biases set: a = silu(c_H) etc., the
    interaction projection and FFN down-projections zero, so u = a + b + c
    and q = w_o . rmsnorm(u) + c_o."""
    T = 4
    P = _zero_params(3, T, 5)
    P["c_H"] = np.full(T, 1.0)
    P["c_E"] = np.array([0.0, 0.0, 2.0, 0.0])
    P["gamma_o"] = np.ones(T)
    P["w_o"] = np.array([[1.0, 0.0, -1.0, 0.0]])
    P["c_o"] = np.array([0.25])
    s1 = 1.0 / (1.0 + math.exp(-1.0))
    s2 = 2.0 / (1.0 + math.exp(-2.0))
    u = np.array([s1, s1, s1 + s2, s1])
    rms = math.sqrt(float(np.mean(u * u)) + 1e-6)
    want = (u[0] - u[2]) / rms + 0.25
    q = recall_score(P, np.ones(3), np.ones(3), np.ones(3))
    assert abs(q - want) < 1e-14


@pytest.mark.parametrize("slot", ["H", "E", "L"])
def test_each_input_feeds_its_own_tower(slot):
    """Only the tower named `slot` is non-zero: the score responds to that
    input alone (h_prev -> H, embedding -> E, local hidden -> L)."""
    D = T = F = 2
    P = _zero_params(D, T, F)
    P[f"gamma_{slot}"] = np.ones(D)
    P[f"W_{slot}"] = np.eye(2)
    P["gamma_o"] = np.ones(T)
    P["w_o"] = np.array([[1.0, -1.0]])
    x = np.array([3.0, -4.0])
    z = np.zeros(2)
    r = x / math.sqrt(12.5 + 1e-6)
    a = r / (1.0 + np.exp(-r))
    want = (a[0] - a[1]) / math.sqrt(float(np.mean(a * a)) + 1e-6)
    args = {"H": (x, z, z), "E": (z, x, z), "L": (z, z, x)}
    for name, inp in args.items():
        q = recall_score(P, *inp)
        if name == slot:
            assert abs(q - want) < 1e-13
        else:
            assert q == 0.0


def test_tower_swap_symmetry():
    """Swapping h_prev <-> h_local together with the H <-> L tower weights and
    the matching interaction columns leaves the score unchanged."""
    D, T, F = 6, 4, 5
    rng = np.random.default_rng(3)
    P = {n: rng.normal(size=s) * 0.5 for n, s in head_layout(D, T, F)}
    x, e, y = rng.normal(size=D), rng.normal(size=D), rng.normal(size=D)
    q1 = recall_score(P, x, e, y)
    P2 = dict(P)
    for k in ("gamma", "W", "c"):
        P2[f"{k}_H"], P2[f"{k}_L"] = P[f"{k}_L"], P[f"{k}_H"]
    # segments [a,b,c,ab,ac,bc,|a-b|,|a-c|,|b-c|] under a<->c become
    # [c,b,a,cb,ca,ba,|c-b|,|c-a|,|b-a|] = segments [2,1,0,5,4,3,8,7,6]
    perm = [2, 1, 0, 5, 4, 3, 8, 7, 6]
    W = P["W_I"].reshape(T, 9, T)
    P2["W_I"] = W[:, perm, :].reshape(T, 9 * T)
    q2 = recall_score(P2, y, e, x)
    assert abs(q1 - q2) < 1e-12


def test_input_scale_invariance():
    """Each tower normalises its input first: scaling an input by a positive
    factor leaves the score unchanged up to the epsilon."""
    D = 2048
    blob = synth.head_blob(D, seed=7, perturb=True)
    P = unpack_head(blob, D)
    rng = np.random.default_rng(9)
    x, e, y = rng.normal(size=D), rng.normal(size=D), rng.normal(size=D)
    q = recall_score(P, x, e, y)
    q2 = recall_score(P, 3.0 * x, 0.5 * e, 10.0 * y)
    # eps = 1e-6 against a mean square near 1 (0.25 after halving) moves the
    # score by a few 1e-6; a missing or misplaced norm moves it by O(1)
    assert abs(q - q2) < 2e-5 * (1 + abs(q))


def test_xavier_init_bounds():
    D = 2048
    blob = synth.head_blob(D, seed=1)
    P = unpack_head(blob, D)
    bound = math.sqrt(6.0 / (1024 + 2048))
    assert np.max(np.abs(P["W_H"])) <= bound and np.max(np.abs(P["W_H"])) > 0.99 * bound
    assert np.all(P["c_I"] == 0) and np.all(P["gamma_1"] == 1)
    assert np.isfinite(recall_score(P, np.ones(D), np.ones(D), np.ones(D)))
