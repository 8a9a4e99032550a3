"""One hybrid block of the Cross-Decoder, decode step, one sequence (test infrastructure only).

ithome page, section "KV Reuse：在同一 Hybrid Block 内，复用 KV 与选择结果": a block is
one full-attention layer followed by several sparse-attention layers; the full
layer selects positions from its attention scores and the sparse layers reuse
its KV cache and its selection indices.  Each sparse layer has its own query
(the layers are distinct); K, V and the indices are identical for all of them
(reading: "reuse the KV cache" means the very same K/V rows, no per-layer
projection).
"""

import numpy as np

from . import attention as _attn
from . import selection as _sel
from . import bf16 as _bf16
from . import e4m3 as _e4m3


def cache_values(data, dtype, scale=None):
    """Stored cache rows -> float64.

    dtype 'f32': float32 array; 'bf16': uint16 bit patterns;
    'e4m3': uint8 codes [..., d] with a float32 scale per row [...].
    """
    if dtype == "f32":
        return np.asarray(data, np.float32).astype(np.float64)
    if dtype == "bf16":
        return _bf16.decode(data)
    if dtype == "e4m3":
        return _e4m3.decode(data) * np.asarray(scale, np.float64)[..., None]
    raise ValueError(dtype)


def full_layer(q, k, v, top_k, window, scale=None, f32_score_keys=False):
    """Full attention + selection for one sequence.

    q [n_q, H, d], k/v [L, n_kv, d] float64.
    Returns dict with o, lse, s (candidate scores), idx, cnt.
    """
    o, lse, p = _attn.full_attention(q, k, v, scale)
    n_kv = k.shape[1]
    s = _attn.selection_scores(p, n_kv, window)
    if f32_score_keys:
        idx, cnt = _sel.select_all(s.astype(np.float32), k.shape[0], top_k, window, True)
    else:
        idx, cnt = _sel.select_all(s, k.shape[0], top_k, window)
    return {"o": o, "lse": lse, "s": s, "idx": idx, "cnt": cnt}


def hybrid_block(q_full, q_sparse, k, v, top_k, window, scale=None):
    """Full layer, then every sparse layer of the block over the same K/V and indices."""
    out = full_layer(q_full, k, v, top_k, window, scale)
    out["sparse"] = [
        _attn.sparse_attention(qs, k, v, out["idx"], out["cnt"], scale)[0] for qs in q_sparse
    ]
    return out
