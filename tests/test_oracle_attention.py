"""Pins of the oracle's attention, score, selection and sparse-attention functions.

Each pin is fixed by something other than the oracle itself: pure-Python brute
force on tiny inputs, torch's float64 scaled_dot_product_attention (a library
routine), closed forms, and invariants the pages state (window always present,
global tokens only from outside it, sparse == full when everything is selected).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention, selection, block

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------- full attention

def _brute_attention(q, k, v, scale):
    """Pure-Python loops: softmax(scale * q.k) weighted sum of v, and log-sum-exp."""
    n_q, H, d = q.shape
    L, n_kv, _ = k.shape
    G = H // n_kv
    o = [[[0.0] * d for _ in range(H)] for _ in range(n_q)]
    lse = [[0.0] * H for _ in range(n_q)]
    for t in range(n_q):
        for h in range(H):
            g = h // G
            logits = [scale * sum(q[t, h, i] * k[j, g, i] for i in range(d)) for j in range(L)]
            m = max(logits)
            w = [math.exp(x - m) for x in logits]
            z = sum(w)
            for i in range(d):
                o[t][h][i] = sum(w[j] * v[j, g, i] for j in range(L)) / z
            lse[t][h] = m + math.log(z)
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("n_q,H,n_kv,L,d", [(1, 1, 1, 1, 3), (2, 4, 1, 7, 5), (3, 4, 2, 6, 4),
                                            (1, 6, 3, 9, 2)])
def test_full_attention_brute_force(n_q, H, n_kv, L, d):
    q = _rand((n_q, H, d), 1)
    k = _rand((L, n_kv, d), 2)
    v = _rand((L, n_kv, d), 3)
    o, lse, p = attention.full_attention(q, k, v, scale=0.7)
    ob, lb = _brute_attention(q, k, v, 0.7)
    assert np.allclose(o, ob, rtol=0, atol=1e-12)
    assert np.allclose(lse, lb, rtol=0, atol=1e-12)
    assert np.allclose(p.sum(axis=2), 1.0, atol=1e-14)


def test_full_attention_vs_torch_sdpa():
    n_q, H, n_kv, L, d = 3, 8, 2, 300, 128
    q = _rand((n_q, H, d), 4)
    k = _rand((L, n_kv, d), 5)
    v = _rand((L, n_kv, d), 6)
    o, lse, _ = attention.full_attention(q, k, v)
    G = H // n_kv
    for g in range(n_kv):
        qt = torch.from_numpy(q[:, g * G:(g + 1) * G, :].reshape(1, 1, n_q * G, d))
        kt = torch.from_numpy(np.ascontiguousarray(k[:, g, :]).reshape(1, 1, L, d))
        vt = torch.from_numpy(np.ascontiguousarray(v[:, g, :]).reshape(1, 1, L, d))
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).numpy().reshape(n_q, G, d)
        assert np.allclose(o[:, g * G:(g + 1) * G], ref, atol=1e-12)
        lref = torch.logsumexp((qt @ kt.transpose(-1, -2)) / math.sqrt(d), dim=-1).numpy()
        assert np.allclose(lse[:, g * G:(g + 1) * G], lref.reshape(n_q, G), atol=1e-12)


def test_full_attention_closed_forms():
    d, L = 128, 513
    q = _rand((2, 4, d), 7)
    # constant V -> o = v
    k = _rand((L, 1, d), 8)
    v = np.tile(_rand((1, 1, d), 9), (L, 1, 1))
    o, _, _ = attention.full_attention(q, k, v)
    assert np.allclose(o, v[0, 0][None, None, :], atol=1e-12)
    # identical K rows -> uniform p, o = mean(V), lse = l + ln L
    k1 = np.tile(_rand((1, 1, d), 10), (L, 1, 1))
    v1 = _rand((L, 1, d), 11)
    o, lse, p = attention.full_attention(q, k1, v1)
    assert np.allclose(p, 1.0 / L, atol=1e-15)
    assert np.allclose(o, v1[:, 0, :].mean(axis=0)[None, None, :], atol=1e-12)
    l0 = (q @ k1[0, 0]) / math.sqrt(d)
    assert np.allclose(lse, l0 + math.log(L), atol=1e-12)
    # L = 1 -> o = v_0, lse = l_0
    o, lse, _ = attention.full_attention(q, k[:1], v[:1] * 0 + v1[:1])
    assert np.allclose(o, v1[0, 0][None, None, :], atol=1e-15)
    assert np.allclose(lse, (q @ k[0, 0]) / math.sqrt(d), atol=1e-12)


def test_needle_dominates():
    """A key 4x along one query's direction (logit ~45) takes all its mass."""
    d, L = 128, 4096
    rng = np.random.default_rng(12)
    q = rng.standard_normal((2, 3, d))
    k = rng.standard_normal((L, 1, d))
    v = rng.standard_normal((L, 1, d))
    p_needle = 1234
    k[p_needle, 0] = 4.0 * q[1, 2]
    o, _, p = attention.full_attention(q, k, v)
    assert p[1, 2, p_needle] > 1 - 1e-9
    assert np.allclose(o[1, 2], v[p_needle, 0], atol=1e-8)


# ---------------------------------------------------------------- selection scores

def test_scores_sum_to_heads_per_group():
    n_q, H, n_kv, L, d = 2, 6, 3, 200, 16
    q, k, v = _rand((n_q, H, d), 13), _rand((L, n_kv, d), 14), _rand((L, n_kv, d), 15)
    _, _, p = attention.full_attention(q, k, v)
    s0 = attention.selection_scores(p, n_kv, window=0)
    assert s0.shape == (n_q, n_kv, L)
    assert np.allclose(s0.sum(axis=2), H // n_kv, atol=1e-12)
    s = attention.selection_scores(p, n_kv, window=17)
    assert s.shape == (n_q, n_kv, L - 17)
    # the window rows are excluded, not dropped from the normalisation
    assert np.allclose(s, s0[:, :, :L - 17], atol=0)


def test_scores_brute_force():
    n_q, H, n_kv, L, d = 2, 4, 2, 9, 3
    q, k, v = _rand((n_q, H, d), 16), _rand((L, n_kv, d), 17), _rand((L, n_kv, d), 18)
    _, _, p = attention.full_attention(q, k, v, scale=1.3)
    s = attention.selection_scores(p, n_kv, window=2)
    G = H // n_kv
    for t in range(n_q):
        for g in range(n_kv):
            for j in range(L - 2):
                ref = 0.0
                for h in range(g * G, (g + 1) * G):
                    lg = [1.3 * sum(q[t, h, i] * k[jj, g, i] for i in range(d)) for jj in range(L)]
                    m = max(lg)
                    ref += math.exp(lg[j] - m) / sum(math.exp(x - m) for x in lg)
                assert abs(s[t, g, j] - ref) < 1e-13


def test_identical_keys_uniform_scores():
    H, L, d = 8, 64, 16
    q = _rand((1, H, d), 19)
    k = np.tile(_rand((1, 1, d), 20), (L, 1, 1))
    _, _, p = attention.full_attention(q, k, _rand((L, 1, d), 21))
    s = attention.selection_scores(p, 1, 0)
    assert np.allclose(s, H / L, atol=1e-14)


# ---------------------------------------------------------------- selection

def test_page_constants_golden():
    g = json.load(open(os.path.join(GOLDEN, "page_constants.json")))
    import synth
    assert synth.WINDOW == g["window"]["value"] == 128
    assert synth.TOP_K == g["global_top_k"]["value"] == 1024
    assert g["global_top_k"]["outside_window"] is True


def _brute_select(scores, L, top_k, window):
    w = min(window, L)
    kk = max(0, min(top_k, L - window))
    order = sorted(range(L - w), key=lambda j: (-scores[j], j))
    return sorted(order[:kk]) + list(range(L - w, L))


@pytest.mark.parametrize("L", [1, 2, 5, 17, 64, 150, 300])
@pytest.mark.parametrize("top_k", [0, 1, 3, 16])
@pytest.mark.parametrize("window", [0, 1, 4])
def test_select_brute_force(L, top_k, window):
    rng = np.random.default_rng(L * 100 + top_k * 10 + window)
    n = L - min(window, L)
    s = rng.integers(0, 7, n).astype(np.float64)       # many ties
    idx, cnt = selection.select(s, L, top_k, window)
    ref = _brute_select(list(s), L, top_k, window)
    assert cnt == len(ref)
    assert list(idx[:cnt]) == ref
    assert np.all(idx[cnt:] == -1)
    assert idx.shape == (top_k + window,)


def test_select_invariants_and_dominance():
    rng = np.random.default_rng(22)
    for L in [127, 128, 129, 1151, 1152, 1153, 5000]:
        n = L - min(128, L)
        s = np.round(rng.random(n) * 50) / 50          # ties
        idx, cnt = selection.select(s, L, 1024, 128)
        w, kk = min(128, L), max(0, min(1024, L - 128))
        assert cnt == min(L, 1152) == w + kk
        sel = idx[:cnt]
        assert np.all(np.diff(sel) > 0)
        assert set(range(L - w, L)) <= set(sel.tolist())         # window always selected
        glob = sel[:kk]
        assert np.all(glob < L - w)                                # globals outside window
        unsel = np.setdiff1d(np.arange(n), glob)
        if kk and unsel.size:
            # every selected a beats every unselected b: s_a > s_b, or equal and a < b
            worst = min(glob, key=lambda a: (s[a], -a))
            best_un = max(unsel, key=lambda b: (s[b], -b))
            assert (s[worst] > s[best_un]) or (s[worst] == s[best_un] and worst < best_un)


def test_select_identical_scores_takes_lowest_indices():
    L = 3000
    idx, cnt = selection.select(np.full(L - 128, 0.25), L, 1024, 128)
    assert list(idx[:1024]) == list(range(1024))
    assert list(idx[1024:cnt]) == list(range(L - 128, L))


def test_f32_key_order_is_float_order():
    rng = np.random.default_rng(23)
    x = np.concatenate([rng.standard_normal(5000) * 10.0 ** rng.integers(-40, 38, 5000),
                        [0.0, -0.0, 1e-45, -1e-45]]).astype(np.float32)
    key = selection.f32_key(x)
    order_key = np.argsort(key, kind="stable")
    xs = x[order_key].astype(np.float64)
    assert np.all(np.diff(xs) >= 0)
    assert selection.f32_key(np.array([-0.0], np.float32))[0] < selection.f32_key(
        np.array([0.0], np.float32))[0]
    with pytest.raises(ValueError):
        selection.f32_key(np.array([np.inf], np.float32))


def test_select_f32_key_mode_matches_brute_force():
    rng = np.random.default_rng(24)
    L = 260
    s = (rng.integers(-3, 4, L - 4) * 0.5).astype(np.float32)
    s[5] = -0.0
    s[6] = 0.0
    idx, cnt = selection.select(s, L, 16, 4, f32_keys=True)
    keys = [int(k) for k in selection.f32_key(s)]
    ref = sorted(sorted(range(L - 4), key=lambda j: (-keys[j], j))[:16]) + list(range(L - 4, L))
    assert list(idx[:cnt]) == ref


# ---------------------------------------------------------------- sparse attention

def test_sparse_equals_full_when_everything_selected():
    rng = np.random.default_rng(25)
    for L in [1, 100, 1152]:
        q = rng.standard_normal((2, 4, 128))
        k = rng.standard_normal((L, 1, 128))
        v = rng.standard_normal((L, 1, 128))
        out = block.hybrid_block(q, [q * 0.5], k, v, 1024, 128)
        assert np.all(out["cnt"] == L)
        assert np.allclose(out["sparse"][0], attention.full_attention(q * 0.5, k, v)[0], atol=1e-12)


def test_sparse_vs_torch_masked_sdpa():
    rng = np.random.default_rng(26)
    n_q, H, L, d = 2, 4, 400, 128
    q = rng.standard_normal((n_q, H, d))
    k = rng.standard_normal((L, 1, d))
    v = rng.standard_normal((L, 1, d))
    idx = np.full((n_q, 1, 40), -1, np.int32)
    cnt = np.array([[33], [40]], np.int32)
    for t in range(n_q):
        idx[t, 0, :cnt[t, 0]] = np.sort(rng.choice(L, cnt[t, 0], replace=False))
    o, _ = attention.sparse_attention(q, k, v, idx, cnt)
    for t in range(n_q):
        mask = torch.zeros(1, 1, H, L, dtype=torch.bool)
        mask[..., idx[t, 0, :cnt[t, 0]]] = True
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[t][None, None]), torch.from_numpy(k[:, 0][None, None]),
            torch.from_numpy(v[:, 0][None, None]), attn_mask=mask).numpy()[0, 0]
        assert np.allclose(o[t], ref, atol=1e-12)


def test_sparse_constant_v():
    rng = np.random.default_rng(27)
    L = 3000
    k = rng.standard_normal((L, 1, 128))
    v = np.tile(rng.standard_normal((1, 1, 128)), (L, 1, 1))
    q = rng.standard_normal((1, 8, 128))
    out = block.hybrid_block(q, [q], k, v, 1024, 128)
    assert np.allclose(out["sparse"][0], v[0, 0][None, None, :], atol=1e-12)
