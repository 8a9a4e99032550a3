"""Sliding-window attention in float64 (test infrastructure only).

ithome page "小米公开 MiMo-V3 核心架构 HySparse2", architecture overview: the
Self-Decoder mixes full attention with sliding-window attention over the
current input, and its full layers' hidden states feed the Cross-Decoder's
KV Bridging.  The pages give neither the window size nor the masking details,
so the plain reading is written out:

* the q_tokens queries are the last q_tokens rows of the sequence's cache (a
  prefill chunk appended before the call): query t sits at position
  pos = L - n_q + t;
* it attends to the band of the w most recent rows up to itself,
  rows max(0, pos - w + 1) .. pos (causal, itself included), with the softmax
  taken over that band only;
* scale 1/sqrt(d) unless given; query head h reads KV head h // (H // n_kv).
"""

import numpy as np

from .attention import _check, default_scale


def band(L, n_q, t, window):
    """Rows [lo, hi] attended by query t of a chunk of n_q at the end of L rows."""
    pos = L - n_q + t
    return max(0, pos - window + 1), pos


def swa_attention(q, k, v, window, scale=None):
    """q [n_q, H, d]; k, v [L, n_kv, d] -> o [n_q, H, d] (one softmax per (token, head) over its band)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n_q, H, d, L, n_kv = _check(q, k, v)
    if window < 1 or n_q > L:
        raise ValueError("window >= 1 and n_q <= L required")
    s = default_scale(d) if scale is None else float(scale)
    G = H // n_kv
    o = np.empty((n_q, H, d))
    for t in range(n_q):
        lo, hi = band(L, n_q, t, window)
        for g in range(n_kv):
            heads = slice(g * G, (g + 1) * G)
            logits = s * (q[t, heads, :] @ k[lo:hi + 1, g, :].T)   # [G, n]
            e = np.exp(logits - logits.max(axis=1, keepdims=True))
            o[t, heads, :] = (e / e.sum(axis=1, keepdims=True)) @ v[lo:hi + 1, g, :]
    return o
