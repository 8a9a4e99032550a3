"""Full attention, selection scores and sparse attention in float64 (test infrastructure only).

Shapes follow the hybrid-block decode step of one sequence:
  q      [n_q, H, d]      query tokens x query heads
  k, v   [L, n_kv, d]     the shared cache rows of this sequence
  group  query head h reads KV head g = h // (H // n_kv)  (MQA: n_kv = 1)

ithome page, section "KV Reuse：在同一 Hybrid Block 内，复用 KV 与选择结果":
a block's full-attention layer attends over the whole shared cache and, while
doing so, picks important positions from its attention scores; the sparse
layers after it read the same cache at those positions.  The pages give no
formula, so the plain textbook softmax attention is written out here.

Readings taken (the pages are silent on each):
* no mask: every query token of the step sees all L cache rows, which already
  hold the current token(s);
* softmax scale 1/sqrt(d) unless the caller passes another;
* "attention scores" used for selection = the full layer's per-head softmax
  probabilities, normalised over all L rows (window included), summed over the
  query heads that share one KV head; one score list per (query token, KV head);
* the sparse layers renormalise the softmax over the selected rows only, with
  no sink and no separate local branch (the separate sliding-window branch is
  removed: ithome page, recent-window paragraphs; ai-bio page, section
  "token 级稀疏与近期 Token 强制窗口").
"""

import numpy as np


def default_scale(d):
    return 1.0 / np.sqrt(float(d))


def _check(q, k, v):
    n_q, H, d = q.shape
    L, n_kv, d2 = k.shape
    if v.shape != k.shape or d2 != d:
        raise ValueError("q/k/v shape mismatch")
    if n_kv < 1 or H % n_kv:
        raise ValueError("n_kv must divide H")
    if L < 1:
        raise ValueError("empty cache")
    return n_q, H, d, L, n_kv


def full_attention(q, k, v, scale=None):
    """Softmax attention of every (token, head) query over all L rows.

    Returns (o [n_q, H, d], lse [n_q, H], p [n_q, H, L]) where
      l_j = scale * <q, k_j>,  m = max_j l_j,  Z = sum_j exp(l_j - m),
      p_j = exp(l_j - m) / Z,  o = sum_j p_j v_j,  lse = m + ln Z.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n_q, H, d, L, n_kv = _check(q, k, v)
    s = default_scale(d) if scale is None else float(scale)
    G = H // n_kv
    o = np.empty((n_q, H, d))
    lse = np.empty((n_q, H))
    p = np.empty((n_q, H, L))
    for g in range(n_kv):
        heads = slice(g * G, (g + 1) * G)
        qg = q[:, heads, :].reshape(n_q * G, d)
        logits = s * (qg @ k[:, g, :].T)                      # [n_q*G, L]
        m = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - m)
        Z = e.sum(axis=1, keepdims=True)
        pg = e / Z
        o[:, heads, :] = (pg @ v[:, g, :]).reshape(n_q, G, d)
        lse[:, heads] = (m + np.log(Z)).reshape(n_q, G)
        p[:, heads, :] = pg.reshape(n_q, G, L)
    return o, lse, p


def selection_scores(p, n_kv, window):
    """Per-(token, KV head) selection scores over the global candidates.

    p [n_q, H, L] are the full layer's probabilities.  The candidates are the
    rows outside the recent window, j in [0, L - W') with W' = min(window, L);
    s[t, g, j] = sum over the heads h of group g of p[t, h, j].
    Returns s [n_q, n_kv, L - W'].
    """
    n_q, H, L = p.shape
    if H % n_kv:
        raise ValueError("n_kv must divide H")
    G = H // n_kv
    w = min(int(window), L)
    return p[:, :, : L - w].reshape(n_q, n_kv, G, L - w).sum(axis=2)


def sparse_attention(q, k, v, idx, count, scale=None):
    """Attention of each (token, head) over its selected rows only.

    idx [n_q, n_kv, C] int (ascending, padded with -1), count [n_q, n_kv].
    The softmax is renormalised over the selected set S:
      o = sum_{j in S} exp(l_j - m_S) v_j / sum_{j in S} exp(l_j - m_S).
    Returns (o [n_q, H, d], lse [n_q, H]).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n_q, H, d, L, n_kv = _check(q, k, v)
    s = default_scale(d) if scale is None else float(scale)
    G = H // n_kv
    o = np.empty((n_q, H, d))
    lse = np.empty((n_q, H))
    for t in range(n_q):
        for g in range(n_kv):
            c = int(count[t, g])
            sel = np.asarray(idx[t, g, :c], dtype=np.int64)
            if c < 1 or sel.min() < 0 or sel.max() >= L:
                raise ValueError("selection out of range")
            ks = k[sel, g, :]
            vs = v[sel, g, :]
            qg = q[t, g * G:(g + 1) * G, :]
            logits = s * (qg @ ks.T)                         # [G, c]
            m = logits.max(axis=1, keepdims=True)
            e = np.exp(logits - m)
            Z = e.sum(axis=1, keepdims=True)
            o[t, g * G:(g + 1) * G, :] = (e / Z) @ vs
            lse[t, g * G:(g + 1) * G] = (m + np.log(Z))[:, 0]
    return o, lse
