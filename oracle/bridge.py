"""KV Bridging: per-target K/V projection of one source hidden state (test infrastructure only).

ithome page, KV-sharing overview (the KV Bridging paragraph): every full
attention layer of the second half (Cross-Decoder) builds its own KV cache from
the *input* hidden state of the matching full layer of the first half
(Self-Decoder); each target layer keeps its own K and V projections, so one
source hidden state yields different K/V per target.  The same is said on the
toolnavs page, section "HySparse2 がやったこと", and on the ai-bio page, section
"两级 KV 共享：KV 桥接与 KV 重用".  Prefill runs only one full-attention layer
(ithome page, prefill early-exit paragraphs), so all targets bridge from the
same source tensor.

Readings taken (the pages give no formula):
* K_l = X W_k,l and V_l = X W_v,l, a plain linear map with no bias, norm or
  rotary embedding;
* bf16 storage: round to nearest even;
* FP8 storage: OCP E4M3FN with one float32 scale per cached row (one token,
  one KV head), separate for K and V: with r the row taken in float32,
  a = max|r_i|, scale = fp32(a / 448) (correctly rounded), scale = 1 when that
  is zero, code_i = e4m3_rne(fp32(r_i / scale)) (correctly rounded division,
  saturating at 448); the stored value is decode(code_i) * scale.
"""

import numpy as np

from . import bf16 as _bf16
from . import e4m3 as _e4m3


def project(x_bits, w_bits):
    """bf16 X [T, D] times bf16 W [D, d] in float64 -> [T, d]."""
    x = _bf16.decode(x_bits)
    w = _bf16.decode(w_bits)
    return x @ w


def quantize_rows_e4m3(r):
    """Rows r [T, d] (any float) -> (codes uint8 [T, d], scale float32 [T])."""
    r32 = np.asarray(r).astype(np.float32)
    a = np.max(np.abs(r32), axis=1)
    scale = (a / np.float32(_e4m3.MAX_FINITE)).astype(np.float32)
    scale = np.where(scale == np.float32(0.0), np.float32(1.0), scale).astype(np.float32)
    y = (r32 / scale[:, None]).astype(np.float32)
    return _e4m3.encode_rne(y), scale


def dequantize_rows_e4m3(codes, scale):
    """codes [T, d], scale [T] -> float64 values (exact)."""
    return _e4m3.decode(codes) * np.asarray(scale, np.float64)[:, None]


def store_bf16(r):
    """Rows r [T, d] float64 -> bf16 bit patterns (RNE)."""
    return _bf16.encode_rne(r)


def bridge(x_bits, w_k_bits, w_v_bits, out_dtype):
    """One source X [T, D] and n targets of (W_k, W_v) [D, d] each.

    Returns a list, one entry per target, of dicts:
      out_dtype 'bf16': {'k': uint16 [T, d], 'v': uint16 [T, d]}
      out_dtype 'e4m3': {'k': uint8 [T, d], 'k_scale': float32 [T], 'v': ..., 'v_scale': ...}
    """
    outs = []
    for wk, wv in zip(w_k_bits, w_v_bits):
        rk = project(x_bits, wk)
        rv = project(x_bits, wv)
        if out_dtype == "bf16":
            outs.append({"k": store_bf16(rk), "v": store_bf16(rv)})
        elif out_dtype == "e4m3":
            kc, ks = quantize_rows_e4m3(rk)
            vc, vs = quantize_rows_e4m3(rv)
            outs.append({"k": kc, "k_scale": ks, "v": vc, "v_scale": vs})
        else:
            raise ValueError(out_dtype)
    return outs
