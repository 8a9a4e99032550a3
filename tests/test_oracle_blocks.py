"""Pins of the oracle's HySparse-v1 block-level selection variant (CPU)."""

import numpy as np
import pytest

from oracle import selection


def _brute(scores, L, top_k, window, block):
    """Pure-Python block selection: sums by loops, sort by (-sum, block)."""
    w = min(window, L)
    kk = max(0, min(top_k, L - window))
    n = L - w
    if kk >= n:
        glob = list(range(n))
    else:
        nb = (n + block - 1) // block
        sums = []
        for b in range(nb):
            t = 0.0
            for j in range(b * block, min(b * block + block, n)):
                t += float(scores[j])
            sums.append(t)
        order = sorted(range(nb), key=lambda b: (-sums[b], b))[:kk // block]
        glob = [j for b in sorted(order) for j in range(b * block, min(b * block + block, n))]
    out = [-1] * (window + top_k)
    out[:len(glob)] = glob
    out[len(glob):len(glob) + w] = list(range(L - w, L))
    return out, len(glob) + w


@pytest.mark.parametrize("L,top_k,window,block", [(200, 64, 16, 8), (300, 128, 0, 16), (1000, 200, 128, 64),
                                                  (1500, 1024, 128, 64), (2000, 256, 128, 64), (1100, 1024, 128, 64),
                                                  (129, 64, 128, 64)])
def test_select_blocks_brute_force(L, top_k, window, block):
    rng = np.random.default_rng(L + top_k + block)
    n = L - min(window, L)
    s = rng.integers(0, 6, n).astype(np.float64) / 4          # many equal block sums -> tie rule
    idx, cnt = selection.select_blocks(s, L, top_k, window, block)
    bidx, bcnt = _brute(s, L, top_k, window, block)
    assert cnt == bcnt and idx.tolist() == bidx


def test_blocks_constant_within_block_rank_by_block_value():
    """Scores constant inside each block: full blocks rank by their value (sum = 64 v), the partial
    last block by (its length x v)."""
    L, W, k = 64 * 40 + 100 + 128, 128, 1024
    n = L - W                                                  # 41 full blocks and one of 36
    nb = (n + 63) // 64
    v = np.random.default_rng(3).permutation(nb).astype(np.float64) + 1.0
    s = np.repeat(v, 64)[:n]
    sums = np.array([v[b] * (min(64 * b + 64, n) - 64 * b) for b in range(nb)])
    want = np.sort(np.argsort(-sums, kind="stable")[:k // 64])
    idx, cnt = selection.select_blocks(s, L, k, W)
    got_blocks = np.unique(idx[:cnt - W] // 64)
    assert np.array_equal(got_blocks, want)


def test_blocks_everything_when_budget_covers_candidates():
    for L in (1, 50, 128, 129, 1152):
        n = L - min(128, L)
        s = np.random.default_rng(L).random(n)
        a = selection.select_blocks(s, L, 1024, 128)
        b = selection.select(s, L, 1024, 128)
        assert a[1] == b[1] and np.array_equal(a[0], b[0])


def test_blocks_budget_and_layout():
    L, W, k = 100000, 128, 1024
    s = np.random.default_rng(9).random(L - W)
    idx, cnt = selection.select_blocks(s, L, k, W)
    g = cnt - W
    assert g == 1024                                           # 16 whole blocks
    glob = idx[:g]
    assert np.all(np.diff(glob) > 0)                           # ascending
    blocks = glob.reshape(16, 64)
    assert np.all(blocks[:, 0] % 64 == 0) and np.all(np.diff(blocks, axis=1) == 1)   # whole aligned blocks
    assert np.array_equal(idx[g:cnt], np.arange(L - W, L)) and np.all(idx[cnt:] == -1)
    # dominance: every chosen block's sum >= every other block's sum
    bs = selection.block_scores(s)
    chosen = blocks[:, 0] // 64
    assert bs[chosen].min() >= np.delete(bs, chosen).max()


def test_f32_tree_order():
    """The float32 tree adds (x0 + x1) + (x2 + x3): here it loses both ones, while a left-to-right
    float32 sum keeps one, and the exact sum is 2."""
    x = np.array([[1e8, 1.0, -1e8, 1.0]], dtype=np.float32)
    assert selection.f32_tree_sum(x)[0] == np.float32(0.0)
    seq = np.float32(0)
    for v in x[0]:
        seq = np.float32(seq + v)
    assert seq == np.float32(1.0)
    # small integers: every partial sum is exact, so the tree equals the exact sum
    m = np.random.default_rng(4).integers(-1000, 1000, (50, 64)).astype(np.float32)
    assert np.array_equal(selection.f32_tree_sum(m), m.astype(np.float64).sum(axis=1).astype(np.float32))


def test_f32_tree_mode_ranks_like_float64_on_exact_sums():
    L, W, k = 64 * 300 + 128, 128, 1024
    s = (np.random.default_rng(5).integers(0, 1 << 10, L - W) / 1024.0).astype(np.float32)
    a = selection.select_blocks(s, L, k, W, f32_tree=True)
    b = selection.select_blocks(s.astype(np.float64), L, k, W)
    assert a[1] == b[1] and np.array_equal(a[0], b[0])
