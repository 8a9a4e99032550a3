"""Sliding-window attention (hs_swa_attn) against the float64 oracle.

Tolerance: 2e-3 max-abs for bf16 caches, 3e-2 for E4M3 caches (the output bounds the method's
parity statement fixes), with the oracle reading the cache and query values exactly as stored."""

import numpy as np
import pytest
import torch

import synth
from oracle import swa
from gpu_cases import Uploaded, banner

pytestmark = pytest.mark.gpu


def _case(kvtype, lens, n_kv, H, n_q, seed):
    rng = np.random.default_rng(seed)
    tot = sum(lens)
    k = rng.standard_normal((tot, n_kv, 128)).astype(np.float32)
    v = rng.standard_normal((tot, n_kv, 128)).astype(np.float32)
    if kvtype == "bf16":                      # stored as bf16 bits; E4M3 caches are quantised from floats
        k, v = synth.bf16_bits(k), synth.bf16_bits(v)
    q = synth.bf16_bits((1.5 * rng.standard_normal((len(lens), n_q, H, 128))).astype(np.float32))
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    case = dict(spec=dict(kv=kvtype, q="bf16"), lengths=np.array(lens), row_start=starts,
                q_full=q, q_sparse=[q], k=k, v=v, needles=[[] for _ in lens])
    return Uploaded(case)


@pytest.mark.parametrize("kvtype,lens,n_kv,H,n_q,w", [
    ("bf16", [300], 1, 32, 300, 128),        # chunk = whole cache: bands grow from 1 row to w
    ("bf16", [517, 250], 1, 32, 200, 100),   # ragged batch, chunk at the end of each cache
    ("e4m3", [517, 250], 1, 32, 200, 100),
    ("bf16", [70], 1, 32, 70, 1000),         # window wider than the cache: causal attention
    ("bf16", [90], 1, 32, 40, 1),            # window 1: the own row's value
    ("e4m3", [400], 2, 64, 37, 33),          # two KV heads, a band of 33 (a one-row last tile)
    ("bf16", [260], 1, 40, 21, 64),          # 40 heads: a partial second block of 32
])
def test_swa_parity(kvtype, lens, n_kv, H, n_q, w):
    banner(f"swa {kvtype} lens={lens} n_kv={n_kv} H={H} n_q={n_q} w={w}")
    from long_context_split_amd import hysparse as hs
    up = _case(kvtype, lens, n_kv, H, n_q, seed=len(lens) * 1000 + w + H)
    B, nq, Hq, _ = up.q_full.shape
    poison = torch.full((B, nq, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    out = hs.swa_attn(up.kv, up.q_full, w, out=poison)     # every element must be written
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    tol = 2e-3 if kvtype == "bf16" else 3e-2
    worst = 0.0
    for i in range(len(lens)):
        q, k, v = up.oracle_seq(i)
        ref = swa.swa_attention(q, k, v, w)
        err = float(np.max(np.abs(got[i] - ref)))
        worst = max(worst, err)
        assert err <= tol, f"sequence {i}: max-abs {err}"
    print(f"[result] swa {kvtype} w={w} max-abs {worst:.2e}", flush=True)


@pytest.mark.parametrize("kvtype,lens,n_kv,H,n_q,w", [
    ("bf16", [517, 250], 1, 32, 200, 100),
    ("e4m3", [400], 2, 64, 37, 33),
    ("bf16", [260], 1, 40, 21, 64),
])
def test_swa_bf16_output(kvtype, lens, n_kv, H, n_q, w):
    """bf16 output (hs_swa_attn_out): bit for bit the float32 call's results rounded to nearest even
    (the oracle's bf16 encoder applied to them), every element written, and within the float32
    tolerance plus half a bf16 step of the float64 oracle."""
    from oracle import bf16
    from long_context_split_amd import hysparse as hs
    banner(f"swa bf16 output {kvtype} lens={lens} n_kv={n_kv} H={H} n_q={n_q} w={w}")
    up = _case(kvtype, lens, n_kv, H, n_q, seed=len(lens) * 1000 + w + H)
    B, nq, Hq, _ = up.q_full.shape
    f32 = hs.swa_attn(up.kv, up.q_full, w)
    poison = torch.full((B, nq, Hq, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    o16 = hs.swa_attn(up.kv, up.q_full, w, out=poison)
    torch.cuda.synchronize()
    bits = o16.view(torch.int16).cpu().numpy().view(np.uint16)
    f32 = f32.cpu().numpy()
    assert np.array_equal(bits, bf16.encode_rne(f32.astype(np.float64)))
    got = bf16.decode(bits)
    tol = 2e-3 if kvtype == "bf16" else 3e-2
    worst = 0.0
    for i in range(len(lens)):
        q, k, v = up.oracle_seq(i)
        ref = swa.swa_attention(q, k, v, w)
        half_step = np.ldexp(1.0, np.frexp(np.abs(ref) + tol)[1] - 9)      # half a bf16 step of |ref| + tol
        excess = float(np.max(np.abs(got[i] - ref) - half_step))
        worst = max(worst, excess)
        assert excess <= tol, f"sequence {i}: max excess over half a bf16 step {excess}"
    print(f"[result] swa bf16-out {kvtype} w={w}: equal to the float32 call rounded; "
          f"max-abs error beyond half a bf16 step {worst:.2e}", flush=True)


@pytest.mark.parametrize("lens,n_kv,H,n_q,w,ring", [
    ([517, 250], 1, 32, 200, 100, "24"),  # 3 groups of 8 per workgroup, a ragged last workgroup
    ([300], 1, 32, 300, 128, "64"),       # bands growing from 1 row; a partial last group
    ([600], 1, 40, 301, 154, "40"),       # widest window the ring holds; a partial second head block
    ([90], 1, 32, 90, 1, "16"),           # window 1
    ([400, 333], 2, 64, 150, 128, "32"),  # two KV heads (32 query heads each), two sequences
    ([2600], 1, 32, 2500, 128, "1"),      # the default split (16 tokens per workgroup here)
    ([2600], 1, 32, 2500, 128, "0"),      # the per-group form on a bf16 cache
])
def test_swa_ring_form(lens, n_kv, H, n_q, w, ring, monkeypatch):
    """bf16 caches: the ring form (tiles at absolute positions in an LDS ring, several 8-token
    groups per workgroup, HS_SWA_RING tokens per workgroup) and the per-group form (HS_SWA_RING=0)
    against the float64 oracle, every element written; the bf16 output equals the float32 one
    rounded to nearest even."""
    from oracle import bf16
    from long_context_split_amd import hysparse as hs
    monkeypatch.setenv("HS_SWA_RING", ring)
    banner(f"swa ring={ring} lens={lens} n_kv={n_kv} H={H} n_q={n_q} w={w}")
    up = _case("bf16", lens, n_kv, H, n_q, seed=len(lens) * 1000 + w + H + 7)
    B, nq, Hq, _ = up.q_full.shape
    out = hs.swa_attn(up.kv, up.q_full, w,
                      out=torch.full((B, nq, Hq, 128), float("nan"), dtype=torch.float32, device="cuda"))
    o16 = hs.swa_attn(up.kv, up.q_full, w,
                      out=torch.full((B, nq, Hq, 128), float("nan"), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    bits = o16.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(bits, bf16.encode_rne(got.astype(np.float64)))
    worst = 0.0
    for i in range(len(lens)):
        q, k, v = up.oracle_seq(i)
        err = float(np.max(np.abs(got[i] - swa.swa_attention(q, k, v, w))))
        worst = max(worst, err)
        assert err <= 2e-3, f"sequence {i}: max-abs {err}"
    print(f"[result] swa ring={ring} w={w} max-abs {worst:.2e}", flush=True)


def test_swa_rejects_bad_arguments():
    from long_context_split_amd import hysparse as hs
    up = _case("bf16", [50], 1, 32, 10, seed=7)
    with pytest.raises(RuntimeError):
        hs.swa_attn(up.kv, up.q_full, 0)                            # window < 1
    q_long = torch.zeros((1, 51, 32, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError):
        hs.swa_attn(up.kv, q_long, 8)                               # more queries than cache rows


@pytest.mark.slow
def test_swa_prefill_chunk_full_size_sampled():
    """A 32768-token chunk over a 32768-row bf16 cache, H = 32, w = 128 (the timed workload); 64
    sampled query tokens against the oracle."""
    banner("swa full size T=32768 H=32 w=128 bf16")
    from long_context_split_amd import hysparse as hs
    T, H, w = 32768, 32, 128
    up = _case("bf16", [T], 1, H, T, seed=11)
    out = hs.swa_attn(up.kv, up.q_full, w)
    torch.cuda.synchronize()
    q, k, v = up.oracle_seq(0)
    rng = np.random.default_rng(12)
    ts = np.unique(np.concatenate([[0, 1, 127, 128, T - 1], rng.integers(0, T, 59)]))
    worst = 0.0
    for t in ts:
        lo = max(0, t - w + 1)
        ref = swa.swa_attention(q[t:t + 1], k[lo:t + 1], v[lo:t + 1], w)[0]
        err = float(np.max(np.abs(out[0, t].cpu().numpy() - ref)))
        worst = max(worst, err)
        assert err <= 2e-3, f"token {t}: max-abs {err}"
    print(f"[result] swa full size max-abs {worst:.2e} over {len(ts)} tokens", flush=True)
