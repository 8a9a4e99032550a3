"""Token-level selection: recent window + top-k global tokens (test infrastructure only).

ithome page, recent-window paragraph under "KV Reuse": the 128 most recent
tokens are always selected and 1,024 global tokens are chosen from outside that
window, both read from the full layer's shared cache.  The same split (window
first, global budget outside it) is stated on the cnyes page, section
"檢索精確到token", and on the toolnavs page, section "HySparse2 がやったこと".
Selection is per token, not per 64-token block (dpshk page, section 03).

Readings taken where the pages are silent:
* W' = min(window, L) rows form the window [L - W', L); the global candidates
  are j in [0, L - W'); the global budget is k' = max(0, min(top_k, L - window));
  when L <= window + top_k every row is selected;
* order of the global candidates: score descending, ties to the lower index;
* emitted list: the k' global indices in ascending order, then the window
  rows in ascending order, padded with -1 up to window + top_k entries;
* on float32 score tensors the order is that of the uint32 key
  bits(x) ^ (0xFFFFFFFF if x is negative else 0x80000000), which is the float
  order for finite values (-0 sorts just below +0); non-finite scores are out
  of contract and rejected.
"""

import numpy as np


def budget(L, top_k, window):
    """(W', k') for a cache of L rows."""
    w = min(int(window), int(L))
    kk = max(0, min(int(top_k), int(L) - int(window)))
    return w, kk


def f32_key(x):
    """float32 scores -> uint32 keys whose unsigned order is the float order."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite score")
    b = x.view(np.uint32)
    neg = (b >> np.uint32(31)) != 0
    return np.where(neg, b ^ np.uint32(0xFFFFFFFF), b ^ np.uint32(0x80000000)).astype(np.uint32)


def _top_global(order_key, kk):
    """Indices of the kk largest keys, ties to the lower index (library sort)."""
    n = order_key.shape[0]
    j = np.arange(n, dtype=np.int64)
    # lexsort: last key is primary -> key descending, then index ascending
    order = np.lexsort((j, -order_key))
    return np.sort(order[:kk])


def select(scores, L, top_k, window, f32_keys=False):
    """Selection list of one (token, KV head).

    scores: the L - W' global-candidate scores (float64, or float32 when
    f32_keys is set, in which case the uint32 key order above is used).
    Returns (idx int32 [window + top_k], count).
    """
    w, kk = budget(L, top_k, window)
    n = int(L) - w
    s = np.asarray(scores)
    if s.shape != (n,):
        raise ValueError(f"expected {n} candidate scores, got {s.shape}")
    if f32_keys:
        key = f32_key(s).astype(np.int64)
    else:
        if not np.all(np.isfinite(s)):
            raise ValueError("non-finite score")
        key = s.astype(np.float64)
    glob = _top_global(key, kk)
    cap = int(window) + int(top_k)
    out = np.full(cap, -1, dtype=np.int32)
    out[:kk] = glob
    out[kk:kk + w] = np.arange(int(L) - w, int(L), dtype=np.int32)
    return out, kk + w


def select_all(s, L, top_k, window, f32_keys=False):
    """select() over s [n_q, n_kv, L - W'] -> (idx [n_q, n_kv, C], count [n_q, n_kv])."""
    n_q, n_kv, _ = s.shape
    cap = int(window) + int(top_k)
    idx = np.empty((n_q, n_kv, cap), dtype=np.int32)
    cnt = np.empty((n_q, n_kv), dtype=np.int32)
    for t in range(n_q):
        for g in range(n_kv):
            idx[t, g], cnt[t, g] = select(s[t, g], L, top_k, window, f32_keys)
    return idx, cnt


# ---------------------------------------------------------------- HySparse v1 block-level variant
#
# dpshk page, section 03, and the cnyes page, section "檢索精確到token": the previous
# HySparse generation chose history in blocks of 64 tokens, so a block with one useful token
# still spent 64 positions of the budget.  Readings taken where the pages are silent:
# * the same scores s_j as the token-level selection, over the same candidates [0, L - W');
# * block b covers candidates [64 b, min(64 b + 64, n)); its score is the sum of its
#   tokens' scores (the block's share of the attention mass);
# * the same token budget: when k' < n, floor(k' / 64) whole blocks are chosen (block
#   score descending, ties to the lower block); when k' >= n every candidate is chosen;
# * emitted list: the chosen blocks' tokens in ascending order, then the window, then -1;
#   count = chosen tokens + W'.

BLOCK = 64


def f32_tree_sum(x):
    """float32 sum of the rows of x [m, 2^p] as a balanced pairwise tree in index order:
    (x0 + x1) + (x2 + x3) ..., every addition rounded to float32.  This is the fixed order in
    which the library's block pooling adds a block's scores, so that tests can take the
    integer block ranking in the same precision on both sides."""
    v = np.ascontiguousarray(x, dtype=np.float32)
    while v.shape[1] > 1:
        v = (v[:, 0::2] + v[:, 1::2]).astype(np.float32)
    return v[:, 0]


def block_scores(scores, block=BLOCK, f32_tree=False):
    """Per-block sums of the candidate scores; the last block may be partial (zeros pad it)."""
    s = np.asarray(scores)
    n = s.shape[0]
    nb = (n + block - 1) // block
    pad = np.zeros(nb * block, dtype=np.float32 if f32_tree else np.float64)
    pad[:n] = s
    m = pad.reshape(nb, block)
    return f32_tree_sum(m) if f32_tree else m.sum(axis=1)


def select_blocks(scores, L, top_k, window, block=BLOCK, f32_tree=False):
    """Block-level selection list of one (token, KV head): (idx int32 [window + top_k], count).
    f32_tree: block sums in the float32 tree order above, ranked by their float32 key order
    (scores must then be float32)."""
    w, kk = budget(L, top_k, window)
    n = int(L) - w
    s = np.asarray(scores)
    if s.shape != (n,):
        raise ValueError(f"expected {n} candidate scores, got {s.shape}")
    cap = int(window) + int(top_k)
    out = np.full(cap, -1, dtype=np.int32)
    if kk >= n:
        glob = np.arange(n, dtype=np.int64)
    else:
        bs = block_scores(s, block, f32_tree)
        key = f32_key(bs).astype(np.int64) if f32_tree else bs.astype(np.float64)
        chosen = _top_global(key, kk // block)             # ascending block indices
        glob = np.concatenate([np.arange(b * block, min(b * block + block, n)) for b in chosen]) \
            if len(chosen) else np.zeros(0, dtype=np.int64)
    g = len(glob)
    out[:g] = glob
    out[g:g + w] = np.arange(int(L) - w, int(L), dtype=np.int32)
    return out, g + w


def select_blocks_all(s, L, top_k, window, block=BLOCK, f32_tree=False):
    """select_blocks() over s [n_q, n_kv, L - W'] -> (idx [n_q, n_kv, C], count [n_q, n_kv])."""
    n_q, n_kv, _ = s.shape
    cap = int(window) + int(top_k)
    idx = np.empty((n_q, n_kv, cap), dtype=np.int32)
    cnt = np.empty((n_q, n_kv), dtype=np.int32)
    for t in range(n_q):
        for g in range(n_kv):
            idx[t, g], cnt[t, g] = select_blocks(s[t, g], L, top_k, window, block, f32_tree)
    return idx, cnt
