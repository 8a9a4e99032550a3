"""Pins of the sliding-window oracle: closed forms, the band edges and the full-attention limit."""

import numpy as np

from oracle import attention, swa


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_window_one_returns_own_value_row():
    rng = np.random.default_rng(1)
    L, n_q, H, n_kv = 40, 9, 6, 2
    q, k, v = _rand(rng, n_q, H, 16), _rand(rng, L, n_kv, 16), _rand(rng, L, n_kv, 16)
    o = swa.swa_attention(q, k, v, 1)
    for t in range(n_q):
        pos = L - n_q + t
        for h in range(H):
            assert np.array_equal(o[t, h], v[pos, h // 3])


def test_equal_keys_give_band_mean():
    rng = np.random.default_rng(2)
    L, n_q, w = 50, 20, 7
    k = np.tile(_rand(rng, 1, 1, 8), (L, 1, 1))
    v = _rand(rng, L, 1, 8)
    q = _rand(rng, n_q, 4, 8)
    o = swa.swa_attention(q, k, v, w)
    for t in range(n_q):
        pos = L - n_q + t
        rows = range(max(0, pos - w + 1), pos + 1)
        mean = sum(v[j, 0] for j in rows) / len(rows)
        assert np.allclose(o[t], mean[None, :], rtol=0, atol=1e-12)


def test_band_edges_with_a_needle():
    """A key far more similar to the query than the rest is taken when it is the band's oldest row and
    ignored one row further back."""
    rng = np.random.default_rng(3)
    L, n_q, w, d = 64, 1, 10, 32
    q = _rand(rng, n_q, 1, d)
    k = 0.01 * _rand(rng, L, 1, d)
    v = _rand(rng, L, 1, d)
    pos = L - 1
    inside, outside = pos - w + 1, pos - w
    k[inside, 0] = (60.0 * np.sqrt(d) / np.dot(q[0, 0], q[0, 0])) * q[0, 0]   # logit 60 against about 0
    o_in = swa.swa_attention(q, k, v, w)[0, 0]
    assert np.allclose(o_in, v[inside, 0], atol=1e-6)
    k2 = k.copy()
    k2[outside] = k[inside]
    k2[inside] = k[inside - 1]
    o_out = swa.swa_attention(q, k2, v, w)[0, 0]
    assert np.linalg.norm(o_out - v[outside, 0]) > 0.5


def test_wide_window_is_full_attention():
    rng = np.random.default_rng(4)
    L, H, n_kv, d = 33, 8, 2, 16
    q, k, v = _rand(rng, 1, H, d), _rand(rng, L, n_kv, d), _rand(rng, L, n_kv, d)
    o_full = attention.full_attention(q, k, v)[0]
    for w in (L, L + 5):
        assert np.allclose(swa.swa_attention(q, k, v, w), o_full, rtol=0, atol=1e-12)


def test_chunk_covering_the_cache_is_causal_attention():
    rng = np.random.default_rng(5)
    L, H, d = 21, 4, 8
    q, k, v = _rand(rng, L, H, d), _rand(rng, L, 1, d), _rand(rng, L, 1, d)
    o = swa.swa_attention(q, k, v, 1000)
    for t in range(L):
        ref = attention.full_attention(q[t:t + 1], k[:t + 1], v[:t + 1])[0][0]
        assert np.allclose(o[t], ref, rtol=0, atol=1e-12)
