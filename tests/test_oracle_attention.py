"""Pins of the oracle's attention (On-Demand Attention notes, section 2.1,
equation for o_t: softmax(q K~[S]^T / sqrt(d_k)) V~[S]).

The oracle is checked against torch's float64 scaled-dot-product attention
(a library routine the index-set attention reduces to once the rows of S are
gathered) and against closed-form special cases.
"""
import math

import numpy as np
import pytest
import torch

from oracle import (attention, decode_attention, full_index_set, kv_group,
                    local_index_set, log_sum_exp_scores)


def _sdpa(q, K, V):
    qt = torch.tensor(q, dtype=torch.float64)[None, None, None, :]
    Kt = torch.tensor(K, dtype=torch.float64)[None, None]
    Vt = torch.tensor(V, dtype=torch.float64)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt)
    return o[0, 0, 0].numpy()


@pytest.mark.parametrize("seed", range(8))
def test_matches_torch_sdpa_on_gathered_rows(seed):
    rng = np.random.default_rng(seed)
    d = int(rng.choice([4, 8, 16, 128]))
    n = int(rng.integers(1, 40))
    K = rng.normal(size=(n, d))
    V = rng.normal(size=(n, d))
    q = rng.normal(size=d) * 2.0
    S = np.sort(rng.choice(n, size=int(rng.integers(1, n + 1)), replace=False))
    got = attention(q, K, V, S)
    want = _sdpa(q, K[S], V[S])
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_single_key_returns_value_exactly():
    rng = np.random.default_rng(1)
    K = rng.normal(size=(5, 8))
    V = rng.normal(size=(5, 8))
    for i in range(5):
        assert np.array_equal(attention(rng.normal(size=8), K, V, [i]), V[i])


def test_zero_query_gives_mean_of_selected_values():
    rng = np.random.default_rng(2)
    K = rng.normal(size=(10, 8))
    V = rng.normal(size=(10, 8))
    S = [0, 3, 4, 9]
    np.testing.assert_allclose(attention(np.zeros(8), K, V, S), V[S].mean(0), rtol=1e-14, atol=1e-14)


def test_uniform_score_shift_changes_nothing():
    """Adding alpha*q/|q|^2 to every key adds alpha/sqrt(d) to every score."""
    rng = np.random.default_rng(3)
    d = 16
    K = rng.normal(size=(12, d))
    V = rng.normal(size=(12, d))
    q = rng.normal(size=d)
    K2 = K + 7.5 * q / np.dot(q, q)
    S = list(range(12))
    np.testing.assert_allclose(attention(q, K, V, S), attention(q, K2, V, S), rtol=1e-12, atol=1e-12)


def test_order_of_index_set_changes_nothing():
    rng = np.random.default_rng(4)
    K = rng.normal(size=(20, 8))
    V = rng.normal(size=(20, 8))
    q = rng.normal(size=8)
    S = np.arange(20)
    np.testing.assert_allclose(attention(q, K, V, S), attention(q, K, V, S[::-1]), rtol=1e-13, atol=1e-14)


def test_dominant_needle():
    """A key whose score exceeds every other by >= 30 takes (almost) all weight."""
    rng = np.random.default_rng(5)
    d = 128
    K = rng.normal(size=(4000, d)) * 0.1
    V = rng.normal(size=(4000, d))
    sigma = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    K[1234] = 1.5 * sigma
    q = 1.5 * sigma
    o = attention(q, K, V, np.arange(4000))
    assert np.max(np.abs(o - V[1234])) < 1e-6


def test_log_sum_exp_matches_torch():
    rng = np.random.default_rng(6)
    K = rng.normal(size=(50, 32))
    q = rng.normal(size=32)
    S = np.arange(0, 50, 3)
    want = torch.logsumexp(torch.tensor(K[S] @ q / math.sqrt(32)), 0).item()
    assert abs(log_sum_exp_scores(q, K, S) - want) < 1e-12


@pytest.mark.parametrize("hq,hkv", [(16, 8), (32, 8), (4, 4), (6, 2)])
def test_gqa_mapping_consecutive_heads_share_kv(hq, hkv):
    """Grouped-query attention: head h reads KV head floor(h / (hq/hkv));
    with hq == hkv it is plain multi-head attention."""
    rng = np.random.default_rng(hq * 100 + hkv)
    d, pos = 8, 9
    q = rng.normal(size=(hq, d))
    Kh = rng.normal(size=(hkv, pos, d)) * np.arange(1, hkv + 1)[:, None, None]
    Vh = rng.normal(size=(hkv, pos, d))
    kc = rng.normal(size=(hkv, d))
    vc = rng.normal(size=(hkv, d))
    S = full_index_set(pos + 1)
    out = decode_attention(q, Kh, Vh, kc, vc, S)
    G = hq // hkv
    for h in range(hq):
        g = h // G
        assert kv_group(h, hq, hkv) == g
        Kt = np.concatenate([Kh[g], kc[g][None]])
        Vt = np.concatenate([Vh[g], vc[g][None]])
        np.testing.assert_allclose(out[h], _sdpa(q[h], Kt, Vt), rtol=1e-12, atol=1e-12)


def test_current_token_comes_from_staging_not_cache():
    """K~_t is the committed history followed by the branch's staged row."""
    rng = np.random.default_rng(7)
    d = 8
    Kh = rng.normal(size=(1, 3, d))
    Vh = rng.normal(size=(1, 3, d))
    kc = rng.normal(size=(1, d))
    vc = rng.normal(size=(1, d))
    q = rng.normal(size=(1, d))
    out = decode_attention(q, Kh, Vh, kc, vc, [3])
    assert np.array_equal(out[0], vc[0])


@pytest.mark.parametrize("t", [1, 2, 5, 100, 2051, 2052])
def test_local_equals_full_bitwise_when_sets_coincide(t):
    """For t <= s + w = 2052 the local and full branch read the same index
    list in the same order, so with identical inputs the oracle's outputs are
    identical bit for bit."""
    rng = np.random.default_rng(t)
    hq, hkv, d = 4, 2, 16
    q = rng.normal(size=(hq, d))
    Kh = rng.normal(size=(hkv, t - 1, d))
    Vh = rng.normal(size=(hkv, t - 1, d))
    kc = rng.normal(size=(hkv, d))
    vc = rng.normal(size=(hkv, d))
    oL = decode_attention(q, Kh, Vh, kc, vc, local_index_set(t))
    oF = decode_attention(q, Kh, Vh, kc, vc, full_index_set(t))
    assert np.array_equal(oL, oF)


def test_local_differs_from_full_after_2052():
    rng = np.random.default_rng(11)
    t, hq, hkv, d = 2053, 2, 1, 8
    q = rng.normal(size=(hq, d))
    Kh = rng.normal(size=(hkv, t - 1, d))
    Vh = rng.normal(size=(hkv, t - 1, d))
    kc, vc = rng.normal(size=(hkv, d)), rng.normal(size=(hkv, d))
    oL = decode_attention(q, Kh, Vh, kc, vc, local_index_set(t))
    oF = decode_attention(q, Kh, Vh, kc, vc, full_index_set(t))
    assert not np.array_equal(oL, oF)
    # the local set is S^F without position 5 (index 4): removing that row
    # from the history makes full attention equal the local one
    Kd = np.delete(Kh, 4, axis=1)
    Vd = np.delete(Vh, 4, axis=1)
    oD = decode_attention(q, Kd, Vd, kc, vc, full_index_set(t - 1))
    np.testing.assert_allclose(oL, oD, rtol=1e-13, atol=1e-14)
